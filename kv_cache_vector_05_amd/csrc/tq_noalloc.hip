// tq_attn_decode_noalloc: the fused decode with its workspace in a static
// device array, for callers that cannot allocate (code under HIP graph
// capture, serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this library's code object: every GPU the library runs
// on holds its own copy until the process ends.  Its device address is taken
// once per device with hipGetSymbolAddress, with that device current, and
// kept; host code passes that address, never the array's name, to the decode.
// Every call on one GPU shares that GPU's array: the decode writes every
// scratch byte it later reads (query digits, split partials, merge stages),
// so nothing has to start at zero, and calls that overlap on one GPU (two
// streams at once) race on it.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "tq_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct Slot {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
Slot g_slots[kMaxDevices];

// device address of this device's scratch array (nullptr and a message on failure)
void* scratch_address(tq_status* st) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *st = tq::hip_fail(e, "hipGetDevice");
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *st = tq::fail(TQ_EUNSUPPORTED, "device index beyond the scratch table");
        return nullptr;
    }
    Slot& s = g_slots[dev];
    std::call_once(s.once, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
    if (s.err != hipSuccess || !s.ptr) {
        *st = tq::hip_fail(s.err != hipSuccess ? s.err : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
        return nullptr;
    }
    return s.ptr;
}

}  // namespace

extern "C" {

tq_status tq_attn_decode_noalloc(const tq_codebook* ck, const tq_codebook* cv, const void* q, int32_t q_dtype,
                                 const tq_packed* k, const tq_packed* v, int32_t B, int32_t Hq, int32_t h_kv,
                                 int32_t L_cap, const int32_t* seq_len, const int32_t* q_pos,
                                 const float* rope_cos, const float* rope_sin, int32_t rope_npos, float scale,
                                 float* out, void* stream) {
    if (!ck || !cv) return tq::fail(TQ_EINVAL, "null codebook");
    const size_t need = tq_workspace_bytes(ck, cv, TQ_OP_DECODE, B, Hq, h_kv, L_cap, 0);
    if (need > kScratchBytes)
        return tq::fail(TQ_EINVAL, "this decode needs " + std::to_string(need) +
                                       " bytes of scratch, above the static maximum of " +
                                       std::to_string(kScratchBytes) + " (use tq_attn_decode with a workspace)");
    tq_status st = TQ_OK;
    void* ws = scratch_address(&st);
    if (!ws) return st;
    return tq_attn_decode(ck, cv, q, q_dtype, k, v, B, Hq, h_kv, L_cap, seq_len, q_pos, rope_cos, rope_sin, rope_npos,
                          scale, out, ws, kScratchBytes, stream);
}

}  // extern "C"
