// noalloc.hip -- dcp_mla_partial_decode_noalloc: the fixed-length MLA decode
// producer with its split partials in a static device array instead of a
// caller-provided scratch buffer, for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops, harnesses that forbid
// hipMalloc).
//
// The array is a file-scope __device__ object: each GPU the library runs on
// gets its own copy, at its own address, when this code object is loaded
// there, and keeps it until the process ends.  In host code the array's name
// is only a stand-in for it, so the address the kernels receive comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept here.
//
// Size: the fixed-length plan gives a shard nsplit > 1 key splits only when
// the (row block, shard) units number base = row_blocks * cp < 256, and then
// nsplit = ceil(256 / base) at most, so nsplit * base <= 256 + base - 1 <=
// 510 units of at most 128 rows, each row 1032 bytes (512 fp16 values, an
// LSE and a scale).  510 * 128 * 1032 bytes therefore hold the partials of
// every shape the entry point accepts; the bound is still checked per call.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "dcp_internal.h"

namespace dcp {
namespace {

constexpr size_t kNoAllocBytes = DCP_NOALLOC_SCRATCH_BYTES;
static_assert(kNoAllocBytes >= size_t{510} * kMlaRowsPerBlock * (kMlaVDim * 2 + 8),
              "the static scratch holds the split partials of every fixed-length shape");

__device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_ptr[kMaxDevices];
std::mutex g_mu;

// Address of `scratch` on device `dev`, which must be the current device.
int scratch_on(int dev, void** out, const char* fn) {
    if (dev < 0 || dev >= kMaxDevices)
        return fail(DCP_ERR_INVALID_ARG, "%s: device %d is beyond the %d this library tracks", fn, dev, kMaxDevices);
    void* p = g_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_mu);
        p = g_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return fail(DCP_ERR_HIP, "%s: hipGetSymbolAddress of the static scratch on device %d failed: %s", fn,
                            dev, hipGetErrorString(e));
            g_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return DCP_OK;
}

}  // namespace
}  // namespace dcp

extern "C" int dcp_mla_partial_decode_noalloc(const void* q, int64_t B, int hq, int64_t q_sb, int64_t q_sh,
                                              const void* kv, int64_t kv_tokens, int64_t kv_st, int dtype, int cp,
                                              float softmax_scale, int lse_mode, void* o_part, int64_t o_sb,
                                              int64_t o_sh, float* lse_part, int64_t lse_sb, void* hip_stream) {
    const char* fn = "dcp_mla_partial_decode_noalloc";
    // The size is checked before any HIP call, so an oversized shape fails
    // the same way on every device.
    size_t need = 0;
    if (B >= 0 && hq >= 1 && kv_tokens >= 0 && cp >= 1 && cp <= DCP_MAX_CP &&
        B * static_cast<int64_t>(hq) <= (int64_t{1} << 30)) {
        int32_t n;
        int64_t len;
        dcp::mla_split(B, hq, kv_tokens, cp, &n, &len, &need);
        if (need > dcp::kNoAllocBytes)
            return dcp::fail(DCP_ERR_WORKSPACE,
                             "%s: this shape needs %zu bytes of split partials but the static scratch holds %zu; "
                             "call dcp_mla_partial_decode with a scratch buffer instead",
                             fn, need, dcp::kNoAllocBytes);
    }
    // The device the kernels run on is the stream's; it must be the current
    // one, with which the array's address is looked up.
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return dcp::fail(DCP_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    if (hip_stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(static_cast<hipStream_t>(hip_stream), &sdev);
        if (e != hipSuccess)
            return dcp::fail(DCP_ERR_STREAM, "%s: hipStreamGetDevice failed: %s", fn, hipGetErrorString(e));
        if (static_cast<int>(sdev) != cur)
            return dcp::fail(DCP_ERR_STREAM,
                             "%s: the stream belongs to device %d but device %d is current; make the stream's "
                             "device current",
                             fn, static_cast<int>(sdev), cur);
    }
    void* ptr = nullptr;
    const int rc0 = dcp::scratch_on(cur, &ptr, fn);
    if (rc0 != DCP_OK) return rc0;
    dcp::MlaPlan plan;
    const int rc = dcp::plan_mla(q, B, hq, q_sb, q_sh, kv, kv_tokens, kv_st, nullptr, dtype, cp, softmax_scale,
                                 lse_mode, o_part, o_sb, o_sh, lse_part, lse_sb, ptr, dcp::kNoAllocBytes, &plan);
    if (rc != DCP_OK) return rc;
    return dcp::run_mla(plan, hip_stream, fn);
}
