// slstm.hip -- the sLSTM cell forward (the scalar-memory cell of xLSTM), gfx950.
//
// Per (batch, head) group of d scalar cells (xLSTM note, section "sLSTM":
// exponential gates with the log-space stabilizer and a normalization; a
// scalar memory with memory mixing), for every token t:
//   pre_g = gx_g,t + R_g h_{t-1}                 g = z, i, f, o; R_g d x d per head
//   m_t   = max(f~ + m_{t-1}, i~)                per cell
//   c_t   = f' c_{t-1} + i' tanh(z~),  n_t = f' n_{t-1} + i'
//   h_t   = sigmoid(o~) c_t / n_t
// with f' = e^{f~ + m_{t-1} - m_t}, i' = e^{i~ - m_t}.
//
// The recurrence is sequential in t and every pre-activation needs all of
// h_{t-1}, so one workgroup owns one group for the whole sequence, and the
// head's four d x d matrices stay in its registers in float32 (256 KiB at
// d = 128: one compute unit's register file) instead of being re-read every
// step.  A wavefront owns 16 cells; its lane (kq, jj) holds the weights of
// all four gates of cell jj for one quarter kq of the inputs, so it reads only
// that quarter of h_{t-1} from LDS (the whole vector per lane would make the
// step LDS-bound), and two cross-lane sums over the quarters leave every lane
// of the cell with its four pre-activations.  Each wavefront then updates its
// own cells; h_t goes to the other half of a double-buffered LDS vector, and
// one barrier per step separates the steps.  The input part gx of each
// pre-activation is loaded a block of PF steps ahead so that the chain of
// steps never waits on memory.
#include <math.h>

#include "common.hpp"
#include "hostcheck.hpp"
#include "mlstm.h"

namespace mlstm {
namespace {

constexpr int PF = 8;  // steps per block of gx loads (even: the h buffers alternate)

template <typename IO>
__device__ __forceinline__ float ld_io(const IO *p) { return to_f(*p); }

// Barrier between two steps.  Only LDS is shared between the wavefronts here
// (h_t is published in LDS; the global store of h_t is read by no other
// wavefront), so this wavefront's LDS operations are waited for and the
// outstanding global loads -- the gx values prefetched for later steps -- are
// not, unlike __syncthreads(), whose fence waits for every memory access.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename IO, int D>
__global__ __launch_bounds__(4 * D) void slstm_kernel(const IO *__restrict__ gx, const IO *__restrict__ R,
                                                      const float *c0, const float *n0, const float *m0,
                                                      const float *h0, IO *__restrict__ hout, float *cT,
                                                      float *nT, float *mT, float *hT, int H, int T) {
    constexpr int KQ = D / 4;  // recurrent inputs per lane
    const int bh = blockIdx.x;
    const int head = bh % H;
    const int tid = threadIdx.x;
    // wavefront w owns cells [16w, 16w + 16); lane (kq, jj) = (lane / 16, lane % 16)
    // holds the four gates' weights of cell 16w + jj for inputs [kq*KQ, (kq+1)*KQ)
    const int lane = tid & 63;
    const int kq = lane >> 4;
    const int j = 16 * (tid >> 6) + (lane & 15);

    __shared__ __attribute__((aligned(16))) float hp[2][D];  // h_{t-1}, double-buffered by step parity

    float r[4][KQ];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const IO *rrow = R + (((size_t)head * 4 + g) * D + j) * D + kq * KQ;
#pragma unroll
        for (int k = 0; k < KQ; ++k) r[g][k] = ld_io(rrow + k);
    }

    // the four lanes of a cell carry its state (they run the same arithmetic
    // on the same values); lane kq == 0 stores it
    float c = 0.0f, n = 0.0f, m = 0.0f;
    const size_t sidx = (size_t)bh * D + j;
    if (c0) {
        c = c0[sidx];
        n = n0[sidx];
        m = m0[sidx];
    }
    if (kq == 0) hp[1][j] = c0 ? h0[sidx] : 0.0f;

    // gx[bh][t][g][j]: lane kq brings in gate kq's input term of step t
    const IO *gp = gx + (size_t)bh * T * 4 * D + kq * D + j;
    IO *hq = hout + (size_t)bh * T * D + j;
    // gx in blocks of PF steps: the raw values of the next block are loaded
    // while the current block runs and converted only when it starts, a whole
    // block after their loads were issued.  Loads go to a clamped step (never
    // a branch around a load: the join would wait for it); the surplus values
    // past T are never used.
    IO xn[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) xn[u] = gp[(size_t)min(u, T - 1) * 4 * D];
    __syncthreads();

    for (int t0 = 0; t0 < T; t0 += PF) {
        float xc[PF];
#pragma unroll
        for (int u = 0; u < PF; ++u) xc[u] = to_f(xn[u]);
#pragma unroll
        for (int u = 0; u < PF; ++u) xn[u] = gp[(size_t)min(t0 + PF + u, T - 1) * 4 * D];
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int t = t0 + u;
            if (t >= T) break;  // uniform
            const float *hprev = hp[(u + 1) & 1] + kq * KQ;   // PF is even: parity of t - 1
            float *hnext = hp[u & 1];
            // partial pre-activations of the four gates over this lane's inputs,
            // two chains per gate; gate kq's input term enters once, here
            float a[4][2];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                a[g][0] = g == kq ? xc[u] : 0.0f;
                a[g][1] = 0.0f;
            }
#pragma unroll
            for (int k = 0; k < KQ; k += 4) {
                const f32x4 hv = *reinterpret_cast<const f32x4 *>(&hprev[k]);
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[g][e & 1] = fmaf(r[g][k + e], hv[e], a[g][e & 1]);
            }
            // sum over the four input quarters (lanes 16 and 32 apart); every
            // lane of the cell ends with the same four values
            float pg[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v = a[g][0] + a[g][1];
                v += __shfl_xor(v, 16, 64);
                v += __shfl_xor(v, 32, 64);
                pg[g] = v;
            }
            const float zt = tanhf(pg[0]);
            const float it = pg[1], ft = pg[2], ot = pg[3];
            const float mn = fmaxf(ft + m, it);
            const float ip = exp_e(it - mn);
            const float fp = exp_e(ft + m - mn);
            c = fmaf(fp, c, ip * zt);
            n = fmaf(fp, n, ip);
            m = mn;
            const float h = sigmoid(ot) * c / n;
            if (kq == 0) {
                hq[(size_t)t * D] = from_f<IO>(h);
                hnext[j] = h;
            }
            // h_t is published; every wavefront is done reading h_{t-1}, whose
            // buffer step t + 1 overwrites
            lds_barrier();
        }
    }
    if (cT && kq == 0) {
        cT[sidx] = c;
        nT[sidx] = n;
        mT[sidx] = m;
        hT[sidx] = hp[(T - 1) & 1][j];
    }
}

template <typename IO>
hipError_t launch_d(int d, int BH, const void *gx, const void *R, const float *c0, const float *n0,
                    const float *m0, const float *h0, void *h, float *cT, float *nT, float *mT, float *hT,
                    int H, int T, hipStream_t s) {
    const IO *g = static_cast<const IO *>(gx);
    const IO *r = static_cast<const IO *>(R);
    IO *ho = static_cast<IO *>(h);
#define SLSTM_CASE(DD)                                                                                \
    case DD:                                                                                          \
        hipLaunchKernelGGL((slstm_kernel<IO, DD>), dim3(BH), dim3(4 * DD), 0, s, g, r, c0, n0, m0, h0, \
                           ho, cT, nT, mT, hT, H, T);                                                 \
        break;
    switch (d) {
        SLSTM_CASE(16)
        SLSTM_CASE(32)
        SLSTM_CASE(48)
        SLSTM_CASE(64)
        SLSTM_CASE(80)
        SLSTM_CASE(96)
        SLSTM_CASE(112)
        SLSTM_CASE(128)
        default:
            return hipErrorInvalidValue;
    }
#undef SLSTM_CASE
    return hipGetLastError();
}

}  // namespace
}  // namespace mlstm

using namespace mlstm;

extern "C" mlstm_status_t mlstm_slstm_fwd(const void *gx, const void *R, const float *c0, const float *n0,
                                          const float *m0, const float *h0, void *h, float *c_T, float *n_T,
                                          float *m_T, float *h_T, int B, int H, int T, int d,
                                          mlstm_dtype_t io, void *stream) {
    if (!gx || !R || !h) return MLSTM_ERR_NULL;
    if (B <= 0 || H <= 0 || T <= 0 || d <= 0) return MLSTM_ERR_SHAPE;
    if (io != MLSTM_F32 && io != MLSTM_BF16) return MLSTM_ERR_UNSUPPORTED;
    if (d % 16 != 0 || d > 128) return MLSTM_ERR_UNSUPPORTED;
    const int nin = (c0 != nullptr) + (n0 != nullptr) + (m0 != nullptr) + (h0 != nullptr);
    const int nout = (c_T != nullptr) + (n_T != nullptr) + (m_T != nullptr) + (h_T != nullptr);
    if ((nin != 0 && nin != 4) || (nout != 0 && nout != 4)) return MLSTM_ERR_STATE_ARGS;
    size_t BH, BHT;
    if (!mul_ok((size_t)B, (size_t)H, &BH) || BH > (size_t)INT32_MAX) return MLSTM_ERR_SHAPE;
    if (!mul_ok(BH, (size_t)T, &BHT) || BHT > ((size_t)1 << 40)) return MLSTM_ERR_SHAPE;
    if (!all_aligned({gx, R, c0, n0, m0, h0, h, c_T, n_T, m_T, h_T})) return MLSTM_ERR_ALIGN;
    const size_t es = io == MLSTM_BF16 ? 2 : 4, ns = BH * d * 4;
    const Range ins[] = {rng(gx, BHT * 4 * d * es), rng(R, (size_t)H * 4 * d * d * es), rng(c0, ns),
                         rng(n0, ns), rng(m0, ns), rng(h0, ns)};
    const Range outs[] = {rng(h, BHT * d * es), rng(c_T, ns), rng(n_T, ns), rng(m_T, ns), rng(h_T, ns)};
    for (int o = 0; o < 5; ++o) {
        for (int i = 0; i < 6; ++i) {
            // a final state may replace its own initial state exactly (in place)
            const bool allowed = o >= 1 && i == o + 1;
            if (overlaps(outs[o], ins[i]) && !(allowed && same(outs[o], ins[i]))) return MLSTM_ERR_ALIAS;
        }
        for (int o2 = o + 1; o2 < 5; ++o2)
            if (overlaps(outs[o], outs[o2])) return MLSTM_ERR_ALIAS;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e =
        io == MLSTM_BF16
            ? launch_d<bf16>(d, (int)BH, gx, R, c0, n0, m0, h0, h, c_T, n_T, m_T, h_T, H, T, s)
            : launch_d<float>(d, (int)BH, gx, R, c0, n0, m0, h0, h, c_T, n_T, m_T, h_T, H, T, s);
    return e == hipSuccess ? MLSTM_OK : MLSTM_ERR_HIP;
}
