// backward.hip -- reverse mode of the mLSTM cell (gradients of a loss whose
// gradient with respect to h is given), gfx950.
//
// Mathematics (xLSTM note, "mLSTM (matrix LSTM)" and "sLSTM" sections, the
// same recurrence as the forward): in the unstabilized variables the
// read-out is C q / max(|n^T q|, 1), so the stabilizer m is not
// differentiated and the gradients are carried in the stabilized variables.
// Per token, with den_t the forward's denominator,
//   a_t    = dh_t * sigmoid(o~_t) / den_t
//   beta_t = -sign(n_t.q_t) (a_t . num_t) / den_t   (0 when the floor is active)
//   dq_t   = C_t a_t + n_t beta_t
//   dk_t   = i'_t (dC*_t v_t + dn*_t),   dv_t = i'_t dC*_t^T k_t
//   do~_t  = dh_t * num_t / den_t * sigmoid'(o~_t)
//   di~_t  = k_t . dk_t,   df~_t = sum_{s >= t} (q_s . dq_s - k_s . dk_s)
// where dC*_t = q_t a_t^T + f'_{t+1} dC*_{t+1} (and dn*_t likewise with
// beta) runs backwards in time with the forward's own decay factors.
//
// Chunkwise, per chunk of L tokens with the forward's in-chunk quantities
// (b = cumsum f~, u_j = i~_j - b_j, r_i = max(m_prev, max_{j<=i} u_j), so
// m_t = b_i + r_i) and the carried gradient G* (stabilized at the chunk's
// last token, m_c = b_{L-1} + r_{L-1}):
//   P_ij  = (q_i.k_j) e^{u_j - r_i},   P~_ij = (a_i.v_j + beta_i) e^{u_j - r_i}   (j <= i)
//   num_i = e^{m_prev - r_i} C'^T q_i + sum_j P_ij v_j     (C', n': state at the chunk start)
//   dq_i  = e^{m_prev - r_i} (C' a_i + n' beta_i) + sum_j P~_ij k_j
//   dk_j  = sum_i P~_ij q_i + w_j (G* v_j + g*),   dv_j = sum_i P_ij a_i + w_j G*^T k_j
//   G*   <- e^{m_prev - r_{L-1}} G* + sum_i e^{m_prev - r_i} q_i a_i^T   (g* likewise)
// with w_j = e^{u_j - r_{L-1}}; after the first chunk G* and g* are the
// gradients of the initial state (C0, n0) and dm0 = <dC0, C0> + dn0 . n0.
//
// Two launches.  The first runs the forward state recurrence per pair and
// stores the state (C', n', m) at every chunk start in the workspace; the
// second walks the chunks backwards.  One workgroup owns one pair.  For
// d_qk, d_v <= 64 it keeps its tiles, the chunk-start state and G* in LDS
// (float32 throughout); larger heads (d_qk <= 256, d_v <= 512) run the same
// steps with them in a per-pair region of the workspace.
#include "common.hpp"

namespace mlstm {

namespace {

constexpr int L = kBwdChunk, D = kBwdMaxDim, NTH = 256;
constexpr int LD = D + 4;  // padded row length of the backward kernel's tiles (floats, 16-byte rows)

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ float hsum(f32x4 x) { return (x[0] + x[1]) + (x[2] + x[3]); }
// sum_r x[r] y[r] over n floats (n a multiple of 4, both 16-byte aligned)
__device__ __forceinline__ float dot(const float *x, const float *y, int n) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int r = 0; r < n; r += 4) acc += ld4(x + r) * ld4(y + r);
    return hsum(acc);
}

// In-chunk gate quantities of tokens t0 .. t0 + L - 1 for the stabilizer
// m_before, by one wavefront (lane j = token j; tokens past T act as i~ =
// -inf, f~ = 0, which leaves every running quantity unchanged):
// gb = cumsum f~, gu = i~ - gb, gr = max(m_before, prefix max gu); last =
// (gb, gr) of the chunk's last token.
__device__ void chunk_gates(const float *ig, const float *fg, int t0, int T, float m_before, float *gb,
                            float *gu, float *gr, float *last) {
    const int lane = threadIdx.x & 63;
    const int t = t0 + lane;
    const bool ok = lane < L && t < T;
    float b = ok ? fg[t] : 0.0f;
    const float i = ok ? ig[t] : -INFINITY;
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(b, o, 64);
        if (lane >= o) b += y;
    }
    const float u = i - b;
    float pm = u;
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(pm, o, 64);
        if (lane >= o) pm = fmaxf(pm, y);
    }
    const float r = fmaxf(m_before, pm);
    if (lane < L) {
        gb[lane] = b;
        gu[lane] = u;
        gr[lane] = r;
    }
    if (lane == L - 1) {
        last[0] = b;
        last[1] = r;
    }
}

template <typename IO>
__global__ __launch_bounds__(NTH) void bwd_ckpt_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) float Cs[D * D], Kt[L * D], Vt[L * D];
    __shared__ float ns[D], wv[L], gb[L], gu[L], gr[L], last[2];
    const int p = blockIdx.x, tid = threadIdx.x;
    const int dk = a.dk, dv = a.dv, T = a.T;
    const int nch = (T + L - 1) / L;
    const size_t rec = (size_t)dk * dv + dk + 1;
    const IO *kg = static_cast<const IO *>(a.k) + (size_t)p * T * dk;
    const IO *vg = static_cast<const IO *>(a.v) + (size_t)p * T * dv;
    const float *igp = a.ig + (size_t)p * T, *fgp = a.fg + (size_t)p * T;

    for (int e = tid; e < dk * dv; e += NTH) Cs[e] = a.C0 ? a.C0[(size_t)p * dk * dv + e] : 0.0f;
    for (int e = tid; e < dk; e += NTH) ns[e] = a.n0 ? a.n0[(size_t)p * dk + e] : 0.0f;
    float m = a.m0 ? a.m0[p] : 0.0f;
    __syncthreads();
    float *ck = a.ckpt + (size_t)p * nch * rec;
    for (int c = 0; c < nch; ++c) {
        const int t0 = c * L;
        float *r = ck + (size_t)c * rec;
        for (int e = tid; e < dk * dv; e += NTH) r[e] = Cs[e];
        for (int e = tid; e < dk; e += NTH) r[(size_t)dk * dv + e] = ns[e];
        if (tid == 0) r[(size_t)dk * dv + dk] = m;
        for (int e = tid; e < L * dk; e += NTH) {
            const int t = t0 + e / dk;
            Kt[e] = t < T ? to_f(kg[(size_t)t * dk + e % dk]) : 0.0f;
        }
        for (int e = tid; e < L * dv; e += NTH) {
            const int t = t0 + e / dv;
            Vt[e] = t < T ? to_f(vg[(size_t)t * dv + e % dv]) : 0.0f;
        }
        if (tid < 64) chunk_gates(igp, fgp, t0, T, m, gb, gu, gr, last);
        __syncthreads();
        const float b_last = last[0], r_last = last[1];
        const float dec = exp_e(m - r_last);
        if (tid < L) wv[tid] = exp_e(gu[tid] - r_last);
        __syncthreads();
        for (int e = tid; e < dk * dv / 4; e += NTH) {
            const int row = (4 * e) / dv, col = (4 * e) % dv;
            f32x4 acc = dec * ld4(&Cs[4 * e]);
#pragma unroll 4
            for (int j = 0; j < L; ++j) acc += (wv[j] * Kt[j * dk + row]) * ld4(&Vt[j * dv + col]);
            *reinterpret_cast<f32x4 *>(&Cs[4 * e]) = acc;
        }
        for (int e = tid; e < dk; e += NTH) {
            float acc = dec * ns[e];
            for (int j = 0; j < L; ++j) acc = fmaf(wv[j], Kt[j * dk + e], acc);
            ns[e] = acc;
        }
        m = b_last + r_last;
        __syncthreads();
    }
}

template <typename IO>
__global__ __launch_bounds__(NTH) void bwd_kernel(BwdArgs a) {
    // rows padded to LD floats: column walks (lanes on consecutive rows) then
    // fall on consecutive banks
    __shared__ __attribute__((aligned(16))) float Q[L * LD], K[L * LD], V[L * LD], SG[L * LD], DH[L * LD],
        NUM[L * LD], A[L * LD], DQ[L * LD], DK[L * LD];
    __shared__ __attribute__((aligned(16))) float Cc[D * LD], Gs[D * LD], P[L * L], PT[L * L];
    __shared__ float nc[D], gs[D], gb[L], gu[L], gr[L], sv[L], fl[L], wv[L], dd[L], den[L], beta[L];
    __shared__ float last[2], carry, red[NTH];
    const int p = blockIdx.x, tid = threadIdx.x;
    const int dk = a.dk, dv = a.dv, T = a.T;
    const int nch = (T + L - 1) / L;
    const size_t rec = (size_t)dk * dv + dk + 1;
    const size_t oqk = (size_t)p * T * dk, ov = (size_t)p * T * dv, og1 = (size_t)p * T;
    const IO *qg = static_cast<const IO *>(a.q) + oqk;
    const IO *kg = static_cast<const IO *>(a.k) + oqk;
    const IO *vg = static_cast<const IO *>(a.v) + ov;
    const IO *ogp = static_cast<const IO *>(a.o) + ov;
    const IO *dhg = static_cast<const IO *>(a.dh) + ov;

    for (int e = tid; e < D * LD; e += NTH) Gs[e] = 0.0f;
    for (int e = tid; e < dk; e += NTH) gs[e] = 0.0f;
    if (tid == 0) carry = 0.0f;
    __syncthreads();
    for (int c = nch - 1; c >= 0; --c) {
        const int t0 = c * L;
        const float *ck = a.ckpt + ((size_t)p * nch + c) * rec;
        for (int e = tid; e < dk * dv; e += NTH) Cc[(e / dv) * LD + e % dv] = ck[e];
        for (int e = tid; e < dk; e += NTH) nc[e] = ck[(size_t)dk * dv + e];
        const float m_prev = ck[(size_t)dk * dv + dk];
        for (int e = tid; e < L * dk; e += NTH) {
            const int i = e / dk, t = t0 + i;
            const size_t g = (size_t)t * dk + e % dk;
            Q[i * LD + e % dk] = t < T ? to_f(qg[g]) : 0.0f;
            K[i * LD + e % dk] = t < T ? to_f(kg[g]) : 0.0f;
        }
        for (int e = tid; e < L * dv; e += NTH) {
            const int i = e / dv, t = t0 + i, x = i * LD + e % dv;
            const size_t g = (size_t)t * dv + e % dv;
            V[x] = t < T ? to_f(vg[g]) : 0.0f;
            SG[x] = t < T ? sigmoid(to_f(ogp[g])) : 0.0f;
            DH[x] = t < T ? to_f(dhg[g]) : 0.0f;
        }
        if (tid < 64) chunk_gates(a.ig + og1, a.fg + og1, t0, T, m_prev, gb, gu, gr, last);
        __syncthreads();
        const float r_last = last[1];
        const float dec = exp_e(m_prev - r_last);
        if (tid < L) {
            sv[tid] = exp_e(m_prev - gr[tid]);
            fl[tid] = exp_e(-(gb[tid] + gr[tid]));
            wv[tid] = exp_e(gu[tid] - r_last);
        }
        // P_ij = (q_i.k_j) e^{u_j - r_i}, causal, rows of real tokens only
        for (int e = tid; e < L * L; e += NTH) {
            const int i = e / L, j = e % L;
            float s = 0.0f;
            if (j <= i && t0 + i < T) s = dot(&Q[i * LD], &K[j * LD], dk) * exp_e(gu[j] - gr[i]);
            P[e] = s;
        }
        __syncthreads();
        // forward read-out and denominator, recomputed
        for (int e = tid; e < L * dv / 4; e += NTH) {
            const int i = (4 * e) / dv, b = (4 * e) % dv;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int r = 0; r < dk; ++r) acc += Q[i * LD + r] * ld4(&Cc[r * LD + b]);
            acc *= sv[i];
            for (int j = 0; j <= i; ++j) acc += P[i * L + j] * ld4(&V[j * LD + b]);
            *reinterpret_cast<f32x4 *>(&NUM[i * LD + b]) = acc;
        }
        if (tid < L) {
            const int i = tid;
            float acc = 0.0f;
            for (int r = 0; r < dk; ++r) acc = fmaf(nc[r], Q[i * LD + r], acc);
            acc *= sv[i];
            for (int j = 0; j <= i; ++j) acc += P[i * L + j];
            dd[i] = acc;
            den[i] = fmaxf(fabsf(acc), fl[i]);
        }
        __syncthreads();
        // a = dh sigmoid(o~) / den, and the output-gate gradient
        for (int e = tid; e < L * dv; e += NTH) {
            const int i = e / dv, x = i * LD + e % dv;
            const float sg = SG[x];
            A[x] = DH[x] * sg / den[i];
            const int t = t0 + i;
            if (t < T) a.go[ov + (size_t)t * dv + e % dv] = DH[x] * NUM[x] / den[i] * sg * (1.0f - sg);
        }
        __syncthreads();
        if (tid < L) {
            const int i = tid;
            const float an = dot(&A[i * LD], &NUM[i * LD], dv);
            beta[i] = fabsf(dd[i]) > fl[i] ? (dd[i] > 0.0f ? -an : an) / den[i] : 0.0f;
        }
        __syncthreads();
        // P~_ij = (a_i.v_j + beta_i) e^{u_j - r_i}
        for (int e = tid; e < L * L; e += NTH) {
            const int i = e / L, j = e % L;
            float s = 0.0f;
            if (j <= i && t0 + i < T) s = (dot(&A[i * LD], &V[j * LD], dv) + beta[i]) * exp_e(gu[j] - gr[i]);
            PT[e] = s;
        }
        __syncthreads();
        for (int e = tid; e < L * dk; e += NTH) {
            const int i = e / dk, r = e % dk;
            float acc = sv[i] * fmaf(nc[r], beta[i], dot(&Cc[r * LD], &A[i * LD], dv));
            for (int j = 0; j <= i; ++j) acc = fmaf(PT[i * L + j], K[j * LD + r], acc);
            DQ[i * LD + r] = acc;
            const int t = t0 + i;
            if (t < T) a.gq[oqk + (size_t)t * dk + r] = acc;
        }
        for (int e = tid; e < L * dk; e += NTH) {
            const int j = e / dk, r = e % dk;
            float acc = 0.0f;
            for (int i = j; i < L; ++i) acc = fmaf(PT[i * L + j], Q[i * LD + r], acc);
            acc = fmaf(wv[j], gs[r] + dot(&Gs[r * LD], &V[j * LD], dv), acc);
            DK[j * LD + r] = acc;
            const int t = t0 + j;
            if (t < T) a.gk[oqk + (size_t)t * dk + r] = acc;
        }
        for (int e = tid; e < L * dv / 4; e += NTH) {
            const int j = (4 * e) / dv, b = (4 * e) % dv;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f}, gk = {0.f, 0.f, 0.f, 0.f};
            for (int i = j; i < L; ++i) acc += P[i * L + j] * ld4(&A[i * LD + b]);
#pragma unroll 4
            for (int r = 0; r < dk; ++r) gk += K[j * LD + r] * ld4(&Gs[r * LD + b]);
            acc += wv[j] * gk;
            const int t = t0 + j;
            if (t < T) *reinterpret_cast<f32x4 *>(&a.gv[ov + (size_t)t * dv + b]) = acc;
        }
        __syncthreads();
        // gate gradients: di = k.dk; df = reverse cumsum of q.dq - k.dk
        if (tid < 64) {
            const int j = tid, t = t0 + j;
            const bool ok = j < L && t < T;
            float di = 0.0f, x = 0.0f;
            if (ok) {
                di = dot(&K[j * LD], &DK[j * LD], dk);
                x = dot(&Q[j * LD], &DQ[j * LD], dk) - di;
            }
            float y = x;  // sum over lanes >= j
            for (int o = 1; o < 64; o <<= 1) {
                const float z = __shfl_down(y, o, 64);
                if (j + o < 64) y += z;
            }
            const float cin = carry;
            if (ok) {
                a.gi[og1 + t] = di;
                a.gf[og1 + t] = y + cin;
            }
            const float tot = __shfl(y, 0, 64);
            if (j == 0) carry = cin + tot;
        }
        // carried gradients for the chunk before (every read of G*, g* is past
        // the barrier above)
        for (int e = tid; e < dk * dv / 4; e += NTH) {
            const int r = (4 * e) / dv, b = (4 * e) % dv;
            f32x4 acc = dec * ld4(&Gs[r * LD + b]);
#pragma unroll 4
            for (int i = 0; i < L; ++i) acc += (sv[i] * Q[i * LD + r]) * ld4(&A[i * LD + b]);
            *reinterpret_cast<f32x4 *>(&Gs[r * LD + b]) = acc;
        }
        for (int e = tid; e < dk; e += NTH) {
            float acc = dec * gs[e];
            for (int i = 0; i < L; ++i) acc = fmaf(sv[i] * beta[i], Q[i * LD + e], acc);
            gs[e] = acc;
        }
        __syncthreads();
    }
    // gradients of the initial state
    float part = 0.0f;
    for (int e = tid; e < dk * dv; e += NTH) {
        const float gx = Gs[(e / dv) * LD + e % dv];
        if (a.gC0) a.gC0[(size_t)p * dk * dv + e] = gx;
        if (a.C0) part = fmaf(gx, a.C0[(size_t)p * dk * dv + e], part);
    }
    for (int e = tid; e < dk; e += NTH) {
        if (a.gn0) a.gn0[(size_t)p * dk + e] = gs[e];
        if (a.n0) part = fmaf(gs[e], a.n0[(size_t)p * dk + e], part);
    }
    red[tid] = part;
    __syncthreads();
    for (int w = NTH / 2; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0 && a.gm0) a.gm0[p] = red[0];
}

// ---- heads above 64: the same two passes with the state, the carried
// gradient and the tiles in a per-pair region of the workspace (global memory,
// served from the caches) instead of LDS, 1024 threads per pair.  Workspace of
// pair p: [nch records of bwd_rec_floats (16-byte aligned)][scratch].

constexpr int NTB = 1024;

template <typename IO>
__global__ __launch_bounds__(NTB) void bwd_ckpt_big_kernel(BwdArgs a) {
    __shared__ float wv[L], gb[L], gu[L], gr[L], last[2];
    const int p = blockIdx.x, tid = threadIdx.x;
    const int dk = a.dk, dv = a.dv, T = a.T;
    const int nch = (T + L - 1) / L;
    const size_t rec = bwd_rec_floats(dk, dv);
    float *ck = a.ckpt + (size_t)p * bwd_ckpt_floats(T, dk, dv);
    float *Kt = ck + (size_t)nch * rec;       // [L][dk], then Vt [L][dv]: the scratch's start
    float *Vt = Kt + (size_t)L * dk;
    const IO *kg = static_cast<const IO *>(a.k) + (size_t)p * T * dk;
    const IO *vg = static_cast<const IO *>(a.v) + (size_t)p * T * dv;
    const float *igp = a.ig + (size_t)p * T, *fgp = a.fg + (size_t)p * T;

    // record 0: the initial state
    for (int e = tid; e < dk * dv; e += NTB) ck[e] = a.C0 ? a.C0[(size_t)p * dk * dv + e] : 0.0f;
    for (int e = tid; e < dk; e += NTB) ck[(size_t)dk * dv + e] = a.n0 ? a.n0[(size_t)p * dk + e] : 0.0f;
    float m = a.m0 ? a.m0[p] : 0.0f;
    if (tid == 0) ck[(size_t)dk * dv + dk] = m;
    // record c + 1 from record c (the state after the last chunk is not needed)
    for (int c = 0; c + 1 < nch; ++c) {
        const int t0 = c * L;
        const float *r = ck + (size_t)c * rec;
        float *r1 = ck + (size_t)(c + 1) * rec;
        for (int e = tid; e < L * dk; e += NTB) {
            const int t = t0 + e / dk;
            Kt[e] = t < T ? to_f(kg[(size_t)t * dk + e % dk]) : 0.0f;
        }
        for (int e = tid; e < L * dv; e += NTB) {
            const int t = t0 + e / dv;
            Vt[e] = t < T ? to_f(vg[(size_t)t * dv + e % dv]) : 0.0f;
        }
        if (tid < 64) chunk_gates(igp, fgp, t0, T, m, gb, gu, gr, last);
        __syncthreads();  // tiles, gates and record c (written by other threads) visible
        const float b_last = last[0], r_last = last[1];
        const float dec = exp_e(m - r_last);
        if (tid < L) wv[tid] = exp_e(gu[tid] - r_last);
        __syncthreads();
        for (int e = tid; e < dk * dv / 4; e += NTB) {
            const int row = (4 * e) / dv, col = (4 * e) % dv;
            f32x4 acc = dec * ld4(&r[4 * e]);
#pragma unroll 4
            for (int j = 0; j < L; ++j) acc += (wv[j] * Kt[j * dk + row]) * ld4(&Vt[j * dv + col]);
            *reinterpret_cast<f32x4 *>(&r1[4 * e]) = acc;
        }
        for (int e = tid; e < dk; e += NTB) {
            float acc = dec * r[(size_t)dk * dv + e];
            for (int j = 0; j < L; ++j) acc = fmaf(wv[j], Kt[j * dk + e], acc);
            r1[(size_t)dk * dv + e] = acc;
        }
        m = b_last + r_last;
        if (tid == 0) r1[(size_t)dk * dv + dk] = m;
        __syncthreads();  // the tiles are rewritten next chunk
    }
}

template <typename IO>
__global__ __launch_bounds__(NTB) void bwd_big_kernel(BwdArgs a) {
    __shared__ float P[L * L], PT[L * L];
    __shared__ float nc_s[kBwdMaxDk], gs[kBwdMaxDk], gb[L], gu[L], gr[L], sv[L], fl[L], wv[L], dd[L],
        den[L], beta[L];
    __shared__ float last[2], carry, red[NTB];
    const int p = blockIdx.x, tid = threadIdx.x;
    const int dk = a.dk, dv = a.dv, T = a.T;
    const int nch = (T + L - 1) / L;
    const size_t rec = bwd_rec_floats(dk, dv);
    const int lk = dk + 4, lv = dv + 4;   // row strides of the dk- and dv-wide tiles
    float *ckp = a.ckpt + (size_t)p * bwd_ckpt_floats(T, dk, dv);
    float *Gs = ckp + (size_t)nch * rec;  // G* [dk][dv]
    float *Q = Gs + (size_t)dk * dv, *K = Q + L * lk, *DQ = K + L * lk, *DK = DQ + L * lk;
    float *V = DK + L * lk, *SG = V + L * lv, *DH = SG + L * lv, *NUM = DH + L * lv, *A = NUM + L * lv;
    const size_t oqk = (size_t)p * T * dk, ov = (size_t)p * T * dv, og1 = (size_t)p * T;
    const IO *qg = static_cast<const IO *>(a.q) + oqk;
    const IO *kg = static_cast<const IO *>(a.k) + oqk;
    const IO *vg = static_cast<const IO *>(a.v) + ov;
    const IO *ogp = static_cast<const IO *>(a.o) + ov;
    const IO *dhg = static_cast<const IO *>(a.dh) + ov;

    for (int e = tid; e < dk * dv; e += NTB) Gs[e] = 0.0f;
    for (int e = tid; e < dk; e += NTB) gs[e] = 0.0f;
    if (tid == 0) carry = 0.0f;
    __syncthreads();
    for (int c = nch - 1; c >= 0; --c) {
        const int t0 = c * L;
        const float *Cc = ckp + (size_t)c * rec;  // C' at the chunk start, rows of dv floats
        for (int e = tid; e < dk; e += NTB) nc_s[e] = Cc[(size_t)dk * dv + e];
        const float m_prev = Cc[(size_t)dk * dv + dk];
        for (int e = tid; e < L * dk; e += NTB) {
            const int i = e / dk, t = t0 + i;
            const size_t g = (size_t)t * dk + e % dk;
            Q[i * lk + e % dk] = t < T ? to_f(qg[g]) : 0.0f;
            K[i * lk + e % dk] = t < T ? to_f(kg[g]) : 0.0f;
        }
        for (int e = tid; e < L * dv; e += NTB) {
            const int i = e / dv, t = t0 + i, x = i * lv + e % dv;
            const size_t g = (size_t)t * dv + e % dv;
            V[x] = t < T ? to_f(vg[g]) : 0.0f;
            SG[x] = t < T ? sigmoid(to_f(ogp[g])) : 0.0f;
            DH[x] = t < T ? to_f(dhg[g]) : 0.0f;
        }
        if (tid < 64) chunk_gates(a.ig + og1, a.fg + og1, t0, T, m_prev, gb, gu, gr, last);
        __syncthreads();
        const float r_last = last[1];
        const float dec = exp_e(m_prev - r_last);
        if (tid < L) {
            sv[tid] = exp_e(m_prev - gr[tid]);
            fl[tid] = exp_e(-(gb[tid] + gr[tid]));
            wv[tid] = exp_e(gu[tid] - r_last);
        }
        for (int e = tid; e < L * L; e += NTB) {
            const int i = e / L, j = e % L;
            float s = 0.0f;
            if (j <= i && t0 + i < T) s = dot(&Q[i * lk], &K[j * lk], dk) * exp_e(gu[j] - gr[i]);
            P[e] = s;
        }
        __syncthreads();
        for (int e = tid; e < L * dv / 4; e += NTB) {
            const int i = (4 * e) / dv, b = (4 * e) % dv;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int r = 0; r < dk; ++r) acc += Q[i * lk + r] * ld4(&Cc[(size_t)r * dv + b]);
            acc *= sv[i];
            for (int j = 0; j <= i; ++j) acc += P[i * L + j] * ld4(&V[j * lv + b]);
            *reinterpret_cast<f32x4 *>(&NUM[i * lv + b]) = acc;
        }
        if (tid < L) {
            const int i = tid;
            float acc = 0.0f;
            for (int r = 0; r < dk; ++r) acc = fmaf(nc_s[r], Q[i * lk + r], acc);
            acc *= sv[i];
            for (int j = 0; j <= i; ++j) acc += P[i * L + j];
            dd[i] = acc;
            den[i] = fmaxf(fabsf(acc), fl[i]);
        }
        __syncthreads();
        for (int e = tid; e < L * dv; e += NTB) {
            const int i = e / dv, x = i * lv + e % dv;
            const float sg = SG[x];
            A[x] = DH[x] * sg / den[i];
            const int t = t0 + i;
            if (t < T) a.go[ov + (size_t)t * dv + e % dv] = DH[x] * NUM[x] / den[i] * sg * (1.0f - sg);
        }
        __syncthreads();
        if (tid < L) {
            const int i = tid;
            const float an = dot(&A[i * lv], &NUM[i * lv], dv);
            beta[i] = fabsf(dd[i]) > fl[i] ? (dd[i] > 0.0f ? -an : an) / den[i] : 0.0f;
        }
        __syncthreads();
        for (int e = tid; e < L * L; e += NTB) {
            const int i = e / L, j = e % L;
            float s = 0.0f;
            if (j <= i && t0 + i < T) s = (dot(&A[i * lv], &V[j * lv], dv) + beta[i]) * exp_e(gu[j] - gr[i]);
            PT[e] = s;
        }
        __syncthreads();
        for (int e = tid; e < L * dk; e += NTB) {
            const int i = e / dk, r = e % dk;
            float acc = sv[i] * fmaf(nc_s[r], beta[i], dot(&Cc[(size_t)r * dv], &A[i * lv], dv));
            for (int j = 0; j <= i; ++j) acc = fmaf(PT[i * L + j], K[j * lk + r], acc);
            DQ[i * lk + r] = acc;
            const int t = t0 + i;
            if (t < T) a.gq[oqk + (size_t)t * dk + r] = acc;
        }
        for (int e = tid; e < L * dk; e += NTB) {
            const int j = e / dk, r = e % dk;
            float acc = 0.0f;
            for (int i = j; i < L; ++i) acc = fmaf(PT[i * L + j], Q[i * lk + r], acc);
            acc = fmaf(wv[j], gs[r] + dot(&Gs[(size_t)r * dv], &V[j * lv], dv), acc);
            DK[j * lk + r] = acc;
            const int t = t0 + j;
            if (t < T) a.gk[oqk + (size_t)t * dk + r] = acc;
        }
        for (int e = tid; e < L * dv / 4; e += NTB) {
            const int j = (4 * e) / dv, b = (4 * e) % dv;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f}, gkv = {0.f, 0.f, 0.f, 0.f};
            for (int i = j; i < L; ++i) acc += P[i * L + j] * ld4(&A[i * lv + b]);
#pragma unroll 4
            for (int r = 0; r < dk; ++r) gkv += K[j * lk + r] * ld4(&Gs[(size_t)r * dv + b]);
            acc += wv[j] * gkv;
            const int t = t0 + j;
            if (t < T) *reinterpret_cast<f32x4 *>(&a.gv[ov + (size_t)t * dv + b]) = acc;
        }
        __syncthreads();
        if (tid < 64) {
            const int j = tid, t = t0 + j;
            const bool ok = j < L && t < T;
            float di = 0.0f, x = 0.0f;
            if (ok) {
                di = dot(&K[j * lk], &DK[j * lk], dk);
                x = dot(&Q[j * lk], &DQ[j * lk], dk) - di;
            }
            float y = x;  // sum over lanes >= j
            for (int o = 1; o < 64; o <<= 1) {
                const float z = __shfl_down(y, o, 64);
                if (j + o < 64) y += z;
            }
            const float cin = carry;
            if (ok) {
                a.gi[og1 + t] = di;
                a.gf[og1 + t] = y + cin;
            }
            const float tot = __shfl(y, 0, 64);
            if (j == 0) carry = cin + tot;
        }
        for (int e = tid; e < dk * dv / 4; e += NTB) {
            const int r = (4 * e) / dv, b = (4 * e) % dv;
            f32x4 acc = dec * ld4(&Gs[(size_t)r * dv + b]);
#pragma unroll 4
            for (int i = 0; i < L; ++i) acc += (sv[i] * Q[i * lk + r]) * ld4(&A[i * lv + b]);
            *reinterpret_cast<f32x4 *>(&Gs[(size_t)r * dv + b]) = acc;
        }
        for (int e = tid; e < dk; e += NTB) {
            float acc = dec * gs[e];
            for (int i = 0; i < L; ++i) acc = fmaf(sv[i] * beta[i], Q[i * lk + e], acc);
            gs[e] = acc;
        }
        __syncthreads();
    }
    float part = 0.0f;
    for (int e = tid; e < dk * dv; e += NTB) {
        const float gx = Gs[e];
        if (a.gC0) a.gC0[(size_t)p * dk * dv + e] = gx;
        if (a.C0) part = fmaf(gx, a.C0[(size_t)p * dk * dv + e], part);
    }
    for (int e = tid; e < dk; e += NTB) {
        if (a.gn0) a.gn0[(size_t)p * dk + e] = gs[e];
        if (a.n0) part = fmaf(gs[e], a.n0[(size_t)p * dk + e], part);
    }
    red[tid] = part;
    __syncthreads();
    for (int w = NTB / 2; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0 && a.gm0) a.gm0[p] = red[0];
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, int io_bf16, hipStream_t s) {
    if (bwd_big(a.dk, a.dv)) {
        dim3 grid(a.BH), block(NTB);
        if (io_bf16) {
            hipLaunchKernelGGL(bwd_ckpt_big_kernel<bf16>, grid, block, 0, s, a);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(bwd_big_kernel<bf16>, grid, block, 0, s, a);
        } else {
            hipLaunchKernelGGL(bwd_ckpt_big_kernel<float>, grid, block, 0, s, a);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(bwd_big_kernel<float>, grid, block, 0, s, a);
        }
        return hipGetLastError();
    }
    dim3 grid(a.BH), block(NTH);
    if (io_bf16) {
        hipLaunchKernelGGL(bwd_ckpt_kernel<bf16>, grid, block, 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(bwd_kernel<bf16>, grid, block, 0, s, a);
    } else {
        hipLaunchKernelGGL(bwd_ckpt_kernel<float>, grid, block, 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(bwd_kernel<float>, grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace mlstm
