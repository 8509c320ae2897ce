// prefill.hip -- instantiations and launchers of the chunkwise forward, and
// the scan that combines per-segment states (segmented schedule).
#include "prefill_bf16.hpp"
#include "prefill_kernel.hpp"
#include "prefill_ws.hpp"

namespace mlstm {

int prefill_dkp(int dk) { return dk <= 32 ? 32 : dk <= 64 ? 64 : dk <= 128 ? 128 : 256; }

int prefill_bv(int io_bf16, int dk, int dv, int chunk) {
    (void)dk; (void)chunk;
    if (io_bf16) return (dv % 128 == 0 || (dv > 128 && dv % 64 != 0)) ? 128 : 64;
    return 64;
}

namespace {

constexpr int kNW = 4;
constexpr size_t kLdsBudget = 160 * 1024;

template <typename IO, int L, int DKP, int BV>
constexpr bool fits() { return PrefillCfg<IO, L, DKP, BV, kNW>::LDS_BYTES <= kLdsBudget; }

template <typename IO, int L, int DKP, int BV, bool SO>
hipError_t run_chunk(const FwdArgs &a, hipStream_t s) {
    if constexpr (fits<IO, L, DKP, BV>()) {
        const int gseg = SO ? a.nseg - 1 : a.nseg;
        dim3 grid((unsigned)(a.BH * gseg * a.ntile)), block(64 * kNW);
        hipLaunchKernelGGL((mlstm_chunk_kernel<IO, L, DKP, BV, kNW, SO>), grid, block, 0, s, a);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

// (chunk, padded d_qk) -> kernel; shapes whose tiles do not fit in LDS are
// rejected by the planner before they get here.
#define MLSTM_SHAPES(X)                                                      \
    X(16, 32) X(16, 64) X(16, 128) X(16, 256) X(32, 32) X(32, 64) X(32, 128) \
    X(32, 256) X(64, 32) X(64, 64) X(64, 128) X(64, 256) X(128, 32) X(128, 64) X(128, 128) X(128, 256)

template <typename IO, int BV, bool SO>
hipError_t by_shape(const FwdArgs &a, int chunk, int dkp, hipStream_t s) {
#define MLSTM_CASE(L_, D_) \
    if (chunk == L_ && dkp == D_) return run_chunk<IO, L_, D_, BV, SO>(a, s);
    MLSTM_SHAPES(MLSTM_CASE)
#undef MLSTM_CASE
    return hipErrorInvalidValue;
}

template <typename IO, int BV>
bool shape_fits(int chunk, int dkp) {
#define MLSTM_CASE(L_, D_) \
    if (chunk == L_ && dkp == D_) return fits<IO, L_, D_, BV>();
    MLSTM_SHAPES(MLSTM_CASE)
#undef MLSTM_CASE
    return false;
}

__global__ __launch_bounds__(256) void seg_combine_kernel(FwdArgs a, const float *local, float *incoming) {
    const int bh = blockIdx.y;
    const int e = blockIdx.x * 256 + threadIdx.x;
    const int dk = a.dk, dv = a.dv;
    const size_t E = (size_t)dk * dv + dk;  // C' then n'
    if ((size_t)e >= E) return;
    const size_t rec = seg_state_floats(dk, dv);
    float m_in = a.m0 ? a.m0[bh] : 0.0f;
    float x;
    if ((size_t)e < (size_t)dk * dv)
        x = a.C0 ? a.C0[(size_t)bh * dk * dv + e] : 0.0f;
    else
        x = a.n0 ? a.n0[(size_t)bh * dk + (e - (size_t)dk * dv)] : 0.0f;
    float *inc = incoming + (size_t)bh * a.nseg * rec;
    inc[e] = x;
    if (e == 0) inc[E] = m_in;
    // (C'_in, m_in) (+) (C'_loc, m_loc, g): the state after a segment whose
    // own contribution, started from nothing, is the local state
    for (int sgi = 0; sgi + 1 < a.nseg; ++sgi) {
        const float *loc = local + ((size_t)bh * (a.nseg - 1) + sgi) * rec;
        const float m_l = loc[E], g = loc[E + 1];
        const float m_new = fmaxf(g + m_in, m_l);
        x = exp_e(g + m_in - m_new) * x + exp_e(m_l - m_new) * loc[e];
        m_in = m_new;
        inc[(size_t)(sgi + 1) * rec + e] = x;
        if (e == 0) inc[(size_t)(sgi + 1) * rec + E] = m_in;
    }
}

}  // namespace

bool bf16_fast_path(int chunk, int dk, int dv);

bool prefill_supported(int io_bf16, int dk, int dv, int chunk) {
    const int dkp = prefill_dkp(dk);
    const int bv = prefill_bv(io_bf16, dk, dv, chunk);
    if (io_bf16 && bf16_fast_path(chunk, dk, dv)) return true;
    if (io_bf16) return bv == 128 ? shape_fits<bf16, 128>(chunk, dkp) : shape_fits<bf16, 64>(chunk, dkp);
    return shape_fits<float, 64>(chunk, dkp);
}

int prefill_kernel_chunk(int io_bf16, int dk, int dv, int chunk) {
    for (int c = chunk; c >= 16; c /= 2)
        if (prefill_supported(io_bf16, dk, dv, c)) return c;
    return 0;
}

// bf16 kernel with LDS copies and transpose reads: chunk <= 64, d_qk in
// {64, 128, 256} (no padding) and d_v a multiple of the column tile
bool bf16_fast_path(int chunk, int dk, int dv) {
    return chunk <= 64 && (dk == 64 || dk == 128 || dk == 256) && dv % 64 == 0;
}

template <int L, int DKP, int BV, bool SO>
hipError_t run_bf16(const FwdArgs &a, hipStream_t s) {
    static_assert(Bf16Cfg<L, DKP, BV>::LDS_BYTES <= kLdsBudget, "LDS budget");
    const int gseg = SO ? a.nseg - 1 : a.nseg;
    dim3 grid((unsigned)(a.BH * gseg * a.ntile)), block(Bf16Cfg<L, DKP, BV>::NTH);
    hipLaunchKernelGGL((mlstm_bf16_kernel<L, DKP, BV, SO>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int BV, bool SO>
hipError_t bf16_by_shape(const FwdArgs &a, int chunk, int dkp, hipStream_t s) {
#define MLSTM_CASE(L_, D_) \
    if (chunk == L_ && dkp == D_) return run_bf16<L_, D_, BV, SO>(a, s);
    MLSTM_CASE(16, 64) MLSTM_CASE(16, 128) MLSTM_CASE(16, 256)
    MLSTM_CASE(32, 64) MLSTM_CASE(32, 128) MLSTM_CASE(32, 256)
    MLSTM_CASE(64, 64) MLSTM_CASE(64, 128) MLSTM_CASE(64, 256)
#undef MLSTM_CASE
    return hipErrorInvalidValue;
}

// role-split kernel: chunk 64, whole 128-column value blocks; the output pass
// or (SO) the segment scan's state-only pass over all segments but the last
template <int DKP, bool SO>
hipError_t run_ws(const FwdArgs &a, hipStream_t s) {
    static_assert(WsCfg<DKP>::LDS_BYTES <= kLdsBudget, "LDS budget");
    const int gseg = SO ? a.nseg - 1 : a.nseg;
    dim3 grid((unsigned)(a.BH * gseg * a.ntile)), block(WsCfg<DKP>::NTH);
    hipLaunchKernelGGL((mlstm_ws_kernel<DKP, SO>), grid, block, 0, s, a);
    return hipGetLastError();
}
template <bool SO>
hipError_t ws_by_shape(const FwdArgs &a, int dkp, hipStream_t s) {
    if (dkp == 256) return run_ws<256, SO>(a, s);
    if (dkp == 128) return run_ws<128, SO>(a, s);
    if (dkp == 64) return run_ws<64, SO>(a, s);
    return hipErrorInvalidValue;
}

bool ws_kernel_selected(int io_bf16, int dk, int dv, int chunk) {
    return io_bf16 && chunk == 64 && prefill_bv(io_bf16, dk, dv, chunk) == 128 && bf16_fast_path(chunk, dk, dv);
}

hipError_t launch_fused(const FwdArgs &a, int io_bf16, int chunk, int state_only, hipStream_t s) {
    const int dkp = prefill_dkp(a.dk);
    const int bv = prefill_bv(io_bf16, a.dk, a.dv, chunk);
    if (ws_kernel_selected(io_bf16, a.dk, a.dv, chunk))
        return state_only ? ws_by_shape<true>(a, dkp, s) : ws_by_shape<false>(a, dkp, s);
    if (io_bf16 && bf16_fast_path(chunk, a.dk, a.dv)) {
        if (bv == 128)
            return state_only ? bf16_by_shape<128, true>(a, chunk, dkp, s)
                              : bf16_by_shape<128, false>(a, chunk, dkp, s);
        return state_only ? bf16_by_shape<64, true>(a, chunk, dkp, s)
                          : bf16_by_shape<64, false>(a, chunk, dkp, s);
    }
    if (io_bf16) {
        if (bv == 128)
            return state_only ? by_shape<bf16, 128, true>(a, chunk, dkp, s)
                              : by_shape<bf16, 128, false>(a, chunk, dkp, s);
        return state_only ? by_shape<bf16, 64, true>(a, chunk, dkp, s)
                          : by_shape<bf16, 64, false>(a, chunk, dkp, s);
    }
    return state_only ? by_shape<float, 64, true>(a, chunk, dkp, s)
                      : by_shape<float, 64, false>(a, chunk, dkp, s);
}

hipError_t launch_seg_combine(const FwdArgs &a, float *ws, hipStream_t s) {
    const size_t E = (size_t)a.dk * a.dv + a.dk;
    const size_t rec = seg_state_floats(a.dk, a.dv);
    float *local = ws;
    float *incoming = ws + (size_t)a.BH * (a.nseg - 1) * rec;
    dim3 grid((unsigned)((E + 255) / 256), (unsigned)a.BH), block(256);
    hipLaunchKernelGGL(seg_combine_kernel, grid, block, 0, s, a, local, incoming);
    return hipGetLastError();
}

}  // namespace mlstm
