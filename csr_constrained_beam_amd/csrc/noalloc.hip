// Allocation-free decoding step (cb_step_noalloc): the same kernels as
// cb_step with the LDS selection, without a plan.  The workspace the dense
// path needs (per-beam candidate keys, full-codebook scores, k-slice partial
// scores, live-beam list) lies in one file-scope device array, so the call
// allocates nothing: for callers that cannot call hipMalloc at call time
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// device allocation).
//
// In host code the array's name is only a host-side stand-in; its device
// address is looked up once per device with hipGetSymbolAddress (each device
// holds its own copy) and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "cb_internal.h"

namespace cb {
namespace {

// 32 MiB: holds the dense path of 2,048 beams over a 2,048-token codebook
// (keys and side information 1 MiB, scores 16 MiB, k-slice partials 4 MiB).
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on `dev` (which is current), looked up on the
// first call on that device.
cb_status scratch_ptr(int dev, unsigned char** out) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            set_error(std::string("cb_step_noalloc: hipGetSymbolAddress of the scratch array failed: ") +
                      hipGetErrorString(e));
            return CB_EHIP;
        }
        g_scratch[dev] = ptr;
    }
    *out = static_cast<unsigned char*>(g_scratch[dev]);
    return CB_OK;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace
}  // namespace cb

using namespace cb;

extern "C" cb_status cb_step_noalloc(const cb_index* idx, int32_t t, int32_t Q, int32_t K, int32_t d, cb_dtype dtype,
                                     cb_path path, const void* hidden, const void* W_t, const int32_t* beam_rows,
                                     const float* acc_logp, int32_t* out_tokens, int32_t* out_parents,
                                     int32_t* out_rows, float* out_logp, void* stream) {
    clear_error();
    if (!idx || idx->device < 0 || idx->device >= kMaxDevices) {
        set_error("cb_step_noalloc: need an index built on a device");
        return CB_EINVAL;
    }
    if (t < 0 || t >= idx->L || Q < 0 || K < 1 || d < 8 || d % 8 || d > 16384 ||
        (dtype != CB_F32 && dtype != CB_BF16) || (int64_t)Q * K >= (int64_t(1) << 31)) {
        set_error("cb_step_noalloc: need 0 <= t < L, Q >= 0, K >= 1, d a multiple of 8 in [8, 16384], "
                  "dtype F32/BF16, Q*K < 2^31");
        return CB_EINVAL;
    }
    if (K > kMaxK) {
        set_error("cb_step_noalloc: beam width above 64 needs the radix selection (cb_step with a plan)");
        return CB_ECAPACITY;
    }
    if (path != CB_PATH_AUTO && path != CB_PATH_DENSE && path != CB_PATH_SPARSE) {
        set_error("cb_step_noalloc: path must be CB_PATH_AUTO, CB_PATH_DENSE or CB_PATH_SPARSE");
        return CB_EINVAL;
    }
    if (Q == 0) return CB_OK;
    const void* vec[] = {hidden, W_t};
    const void* per[] = {beam_rows, acc_logp, out_tokens, out_parents, out_rows, out_logp};
    for (const void* x : vec)
        if (!x || !aligned(x, 16)) {
            set_error("cb_step_noalloc: hidden or W_t is NULL or not 16-byte aligned");
            return CB_EINVAL;
        }
    for (const void* x : per)
        if (!x || !aligned(x, 4)) {
            set_error("cb_step_noalloc: a per-slot array is NULL or not 4-byte aligned");
            return CB_EINVAL;
        }
    const size_t R = (size_t)Q * K;
    void* const outs[4] = {out_tokens, out_parents, out_rows, out_logp};
    if (step_args_alias(R, (size_t)d, (size_t)idx->V, dtype, hidden, W_t, beam_rows, acc_logp, outs)) {
        set_error("cb_step_noalloc: an output array overlaps an input or another output");
        return CB_EINVAL;
    }
    const StepTable& T = idx->steps[(size_t)t];
    const bool dense_ok = dtype == CB_F32 || d % 64 == 0;
    int32_t p = path;
    if (p == CB_PATH_AUTO) p = (T.store == CB_STORE_BITMAP && dense_ok) ? CB_PATH_DENSE : CB_PATH_SPARSE;
    if (p == CB_PATH_DENSE && !dense_ok) {
        set_error("cb_step_noalloc: the dense path needs d to be a multiple of 64 for bf16");
        return CB_EUNSUPPORTED;
    }
    const int Kc = std::min(K, std::max(T.S, 1));
    // the LDS selection must hold the step (as for a plan's CB_SELECT_LDS)
    const bool fits = expand_lds_bytes(T.S, d, true) <= (size_t)kMaxLds &&
                      (p == CB_PATH_DENSE || (d <= kQueryMaxD ? query_lds_bytes(T.S, K, Kc, d) <= (size_t)kMaxLds
                                                              : expand_lds_bytes(T.S, d, false) <= (size_t)kMaxLds));
    if (!fits) {
        set_error("cb_step_noalloc: a row of this step is too wide for the LDS selection (use cb_step with a plan)");
        return CB_ECAPACITY;
    }
    // workspace: per-beam keys and their side information on the dense path
    // and on the wide-hidden sparse route; full-codebook scores, k-slice
    // partials and the live list on the dense path; none for the fused
    // per-query sparse step
    const bool need_keys = p == CB_PATH_DENSE || d > kQueryMaxD;
    const bool need_dense = p == CB_PATH_DENSE;
    const size_t b_keys = need_keys ? 2 * round256(R * Kc * 8) : 0;
    const size_t b_z = need_dense ? round256(R * (size_t)idx->V * 4) : 0;
    const size_t b_zp = need_dense && dtype == CB_BF16 ? round256(split_scores_floats(idx->V) * 4) : 0;
    const size_t b_live = need_dense ? 2 * round256(R * 4) + 256 : 0;
    const size_t need = b_keys + b_z + b_zp + b_live;
    if (need > kScratchBytes) {
        set_error("cb_step_noalloc: this step needs " + std::to_string(need) + " bytes of workspace, above the " +
                  std::to_string(kScratchBytes) + "-byte static array (use cb_step with a plan)");
        return CB_ECAPACITY;
    }
    DeviceGuard g(idx->device);
    if (!g.ok) {
        set_error("cb_step_noalloc: cannot select the index's device");
        return CB_EHIP;
    }
    unsigned char* base = nullptr;
    cb_status st = scratch_ptr(idx->device, &base);
    if (st != CB_OK) return st;
    // a plan on the stack whose workspace pointers lie in the array (its
    // containers stay empty; nothing is allocated or freed)
    cb_plan w;
    w.idx = const_cast<cb_index*>(idx);
    w.device = idx->device;
    w.Q_max = Q;
    w.K = K;
    w.d = d;
    w.dtype = dtype;
    w.Kc_max = Kc;
    unsigned char* cur = base;
    if (b_keys) {
        w.keys = reinterpret_cast<uint64_t*>(cur);
        w.side = reinterpret_cast<uint64_t*>(cur + b_keys / 2);
        cur += b_keys;
    }
    if (need_dense) {
        w.Z = reinterpret_cast<float*>(cur);
        cur += b_z;
        if (b_zp) {
            w.Zp = reinterpret_cast<float*>(cur);
            cur += b_zp;
        }
        w.live = reinterpret_cast<int32_t*>(cur);
        cur += round256(R * 4);
        w.ci_of = reinterpret_cast<int32_t*>(cur);
        cur += round256(R * 4);
        w.n_live = reinterpret_cast<int32_t*>(cur);
    }
    return enqueue_step(&w, t, Q, p, CB_SELECT_LDS, hidden, W_t, beam_rows, acc_logp, out_tokens, out_parents,
                        out_rows, out_logp, (hipStream_t)stream);
}
