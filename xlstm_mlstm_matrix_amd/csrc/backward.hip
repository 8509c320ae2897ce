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
// Five launches (d_qk <= 256, d_v <= 512): a checkpoint pass stores the
// state (C', n', m) at every chunk start, and chunk-parallel passes and
// column-block scans take the gradients from there (the section "the passes"
// below).  A single workgroup per pair walking the chunks backwards leaves
// the chip idle at small batch and cannot hold heads above 64 in LDS; the
// passes have B*H*(T/L) workgroups in their chunk-parallel launches.
#include "common.hpp"

namespace mlstm {

namespace {

constexpr int L = kBwdChunk;

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ float hsum(f32x4 x) { return (x[0] + x[1]) + (x[2] + x[3]); }
// sum_r x[r] y[r] over n floats (n a multiple of 4, both 16-byte aligned)
__device__ __forceinline__ float dot(const float *x, const float *y, int n) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int r = 0; r < n; r += 4) acc += ld4(x + r) * ld4(y + r);
    return hsum(acc);
}

// In-chunk gate quantities of one chunk for the stabilizer m_before, by one
// wavefront (lane j = token j, given its f~ and i~; tokens past T and lanes
// past L act as i~ = -inf, f~ = 0, which leaves every running quantity
// unchanged): gb = cumsum f~, gu = i~ - gb, gr = max(m_before, prefix max
// gu); last = (gb, gr) of the chunk's last token.  Returns the lane's (u, r).
__device__ void gate_scan(float b, float i, float m_before, float *gb, float *gu, float *gr, float *last,
                          float *u_out, float *r_out) {
    const int lane = threadIdx.x & 63;
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
    *u_out = u;
    *r_out = r;
}

// The part of gate_scan that does not depend on the stabilizer: lane j's
// cumsum b of f~, u = i~ - b and the prefix max pm of u over lanes <= j.
__device__ __forceinline__ void gate_prefix(float f, float i, float *b_out, float *u_out, float *pm_out) {
    const int lane = threadIdx.x & 63;
    float b = f;
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
    *b_out = b;
    *u_out = u;
    *pm_out = pm;
}

// gate_scan of tokens t0 .. t0 + L - 1, loading their gates
__device__ void chunk_gates(const float *ig, const float *fg, int t0, int T, float m_before, float *gb,
                            float *gu, float *gr, float *last) {
    const int lane = threadIdx.x & 63;
    const int t = t0 + lane;
    const bool ok = lane < L && t < T;
    float u, r;
    gate_scan(ok ? fg[t] : 0.0f, ok ? ig[t] : -INFINITY, m_before, gb, gu, gr, last, &u, &r);
}

// ---- the passes.  Only the carried gradient G* is sequential over chunks:
// everything else of a chunk follows from its checkpointed state.  So, after
// the checkpoint pass:
//   A (pair, chunk): P, the read-out, a, beta, P~ and do~            -> workspace
//   B (pair, BVB value columns): the reverse scan of G*, g* over the chunks,
//     storing the value entering every chunk; dC0, dn0 and dm0 partials
//   C (pair, chunk): dq, dk, dv, di~ and the in-chunk part of df~
//   D (pair): df~'s carry across chunks and dm0
// Tiles live in LDS in float32; the state, a, G* come from the workspace
// through the caches.  Workspace layout: bwd_layout.

// value columns per workgroup of the two scans (128 measured fastest when the
// scans ran on the vector units: 64 and 32 re-read the K or Q tile more
// often, 256 halves the workgroups), and their threads (eight wavefronts, each
// holding two 16-row tiles of the block by two 64-column quads as MFMA
// accumulators; rows up to 256)
constexpr int NTA = 512, BVB = 128, CG = BVB / 16, NTS = 64 * CG;

// load rows t0 .. t0 + L - 1 of a [T, d] input as float32 into a [L][ld] tile
// (zero past T)
template <typename IO>
__device__ __forceinline__ void load_tile(float *dst, int ld, const IO *src, int d, int t0, int T, int tid,
                                          int nt) {
    for (int e = tid; e < L * d; e += nt) {
        const int i = e / d, t = t0 + i;
        dst[i * ld + e % d] = t < T ? to_f(src[(size_t)t * d + e % d]) : 0.0f;
    }
}
template <typename IO>
__device__ __forceinline__ f32x4 ld4_io(const IO *p) {
    return f32x4{to_f(p[0]), to_f(p[1]), to_f(p[2]), to_f(p[3])};
}

// Barrier for the two scans.  Within them only LDS is shared between the
// wavefronts (their global stores are read by later launches), so this waits
// for this wavefront's LDS operations and not for the outstanding global
// loads of the next chunk, unlike __syncthreads(), whose fence waits for
// every memory access.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Buffer descriptor over nbytes from p (32-bit data format, default cache
// policy).  Loads at offsets past nbytes return zero without touching memory.
constexpr int kBufFlags = 0x00020000;
constexpr unsigned kFar = 0x80000000u;  // an offset past every buffer here (nbytes <= 2^31)
template <typename E>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const E *p, size_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<E *>(p), 0, (int)nbytes, kBufFlags);
}

// Four consecutive elements, loaded in one instruction and converted later.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <typename E> struct Quad;
template <> struct Quad<float> {
    typedef f32x4 raw;
    static __device__ __forceinline__ raw load(__amdgpu_buffer_rsrc_t r, unsigned off) {
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    }
    static __device__ __forceinline__ f32x4 cvt(raw x) { return x; }
};
template <> struct Quad<bf16> {
    typedef bf16x4 raw;
    static __device__ __forceinline__ raw load(__amdgpu_buffer_rsrc_t r, unsigned off) {
        return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
    }
    static __device__ __forceinline__ f32x4 cvt(raw x) {
        return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
    }
};

// Rows t0 .. t0 + L - 1, columns [c0, c0 + w) of a row-major tensor with ld
// elements per row, staged through registers in groups of four: fetch()
// issues the loads of one chunk, put() converts them to float32 and writes
// them to an [L][ldd] LDS tile.  Rows past the descriptor's end (tokens past
// T) read as zero; groups past the tile (NQ * NT may exceed L * w / 4) load
// nothing and are not written; whole rounds of NT groups past the tile are
// skipped.  w and c0 are multiples of 4.
template <typename E, int NQ, int NT>
struct TileFetch {
    typename Quad<E>::raw r[NQ];
    __device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t rs, int ld, int c0, int w, int t0, int tid) {
        const int g4 = w >> 2;
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            if (u * NT >= L * g4) break;  // uniform: no group of this round lies in the tile
            const int q = tid + u * NT, i = q / g4;
            const unsigned e = (unsigned)(t0 + i) * (unsigned)ld + (unsigned)(c0 + 4 * (q - i * g4));
            r[u] = Quad<E>::load(rs, i < L ? e * (unsigned)sizeof(E) : kFar);
        }
    }
    // dst holds L * ldd floats and one spare group after them, which takes
    // the surplus groups (no branch: a store skipped on some lanes would
    // leave its loads unwaited on that path, and the compiler's merged wait
    // counts would then also wait for the stores issued after them)
    __device__ __forceinline__ void put(float *dst, int ldd, int w, int tid) const {
        const int g4 = w >> 2;
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            if (u * NT >= L * g4) break;  // uniform, as in fetch
            const int q = tid + u * NT, i = q / g4;
            *reinterpret_cast<f32x4 *>(&dst[i < L ? i * ldd + 4 * (q - i * g4) : L * ldd]) = Quad<E>::cvt(r[u]);
        }
    }
};

// 16- and 4-byte buffer accesses of float32 data (stores past the
// descriptor's end are dropped, loads there return zero)
__device__ __forceinline__ f32x4 buf_ld4(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ void buf_st4(f32x4 x, __amdgpu_buffer_rsrc_t r, unsigned off) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_st1(float x, __amdgpu_buffer_rsrc_t r, unsigned off) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), r, (int)off, 0, 0);
}

// v_mfma_f32_16x16x4_f32: D[16][16] += A[16][4] B[4][16], float32 products
// and sums.  Lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] and
// holds D[4 (l / 16) + v][l % 16] in element v.
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Products [L tokens] x [rows of a record] x [64 value columns] (passes A and
// C): four steps of record rows (steps sc .. sc + 3, rows 4s + g, sc =
// min(s0, ns - 4)) into gr4, and their MFMAs against a token tile in LDS
// (on = 0 makes a group contribute nothing).
__device__ __forceinline__ void dv_gload(f32x4 (&gr4)[4], __amdgpu_buffer_rsrc_t r, unsigned off,
                                         unsigned rstep, int s0, int ns) {
    const int sc = min(s0, ns - 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) gr4[u] = buf_ld4(r, off + (unsigned)(sc + u) * rstep);
}
template <int LK>
__device__ __forceinline__ void dv_gstep(f32x4 (&x)[2][4], const f32x4 (&gr4)[4], const float *K, int l16, int g,
                                         int s0, float on) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = 4 * (s0 + u) + g;
        const float k0 = on * K[l16 * LK + r], k1 = on * K[(16 + l16) * LK + r];
#pragma unroll
        for (int xx = 0; xx < 4; ++xx) {
            x[0][xx] = mfma4(k0, gr4[u][xx], x[0][xx]);
            x[1][xx] = mfma4(k1, gr4[u][xx], x[1][xx]);
        }
    }
}

// Checkpoint pass: one workgroup per (block of BVB value columns, pair).  The
// state recurrence is separable by value column, so each workgroup carries
// its [d_qk][BVB] block of C' in registers (as MFMA accumulators, laid out
// below) and writes it to the record of every chunk start; block 0 also
// carries n' and writes m (every block computes the same gates).  The K and V
// tiles and the gates of the next chunk load while the current chunk
// computes.
template <typename IO>
__global__ __launch_bounds__(NTS) void bwd_ckpt_kernel(BwdArgs a) {
    constexpr int LK = kBwdMaxDk + 4;
    __shared__ __attribute__((aligned(16))) float Ks[L * LK + 4], Vs[L * BVB + 4];
    __shared__ float ns[kBwdMaxDk], wv[L], last[2];
    const int blk = blockIdx.x, p = blockIdx.y, tid = threadIdx.x;
    const int dk = a.dk, dv = a.dv, T = a.T;
    const int c0 = blk * BVB, w = min(BVB, dv - c0);
    const BwdLayout lay = bwd_layout(T, dk, dv);
    const int nch = (int)lay.nch;
    const size_t rec = lay.rec;
    float *base = a.ckpt + (size_t)p * lay.total;
    const IO *kg = static_cast<const IO *>(a.k) + (size_t)p * T * dk;
    const IO *vg = static_cast<const IO *>(a.v) + (size_t)p * T * dv;
    const float *igp = a.ig + (size_t)p * T, *fgp = a.fg + (size_t)p * T;
    const __amdgpu_buffer_rsrc_t kr = rsrc(kg, (size_t)T * dk * sizeof(IO));
    const __amdgpu_buffer_rsrc_t vr = rsrc(vg, (size_t)T * dv * sizeof(IO));
    TileFetch<IO, L * kBwdMaxDk / 4 / NTS, NTS> kf;
    TileFetch<IO, L * BVB / 4 / NTS, NTS> vf;
    auto fetch = [&](int t0) {
        kf.fetch(kr, dk, 0, dk, t0, tid);
        vf.fetch(vr, dv, c0, w, t0, tid);
    };
    fetch(0);
    // The gates: every lane loads those of token t0 + lane % 64 (clamped into
    // the sequence) two chunks ahead, into (ni, nf).  They are scanned a chunk
    // ahead into (sb, su, sp) (gate_prefix), and the scan is finished with the
    // stabilizer when the chunk starts; only last[] and wv[] are read by the
    // other wavefronts.  When the last wavefront holds no state tiles (d_qk up
    // to 112) it alone does this, while the others run the chunk's MFMAs;
    // otherwise every wavefront does (one would delay the chunk).
    const int lane = tid & 63;
    const bool gwave = 16 * (NTS / 64 - 1) >= dk ? (tid >> 6) == NTS / 64 - 1 : true;
    float ni, nf, sb = 0.0f, su = 0.0f, sp = 0.0f;
    auto gload = [&](int t0) {
        const int t = min(t0 + lane, T - 1);
        ni = igp[t];
        nf = fgp[t];
    };
    auto gscan = [&](int t0) {
        const bool ok = lane < L && t0 + lane < T;
        gate_prefix(ok ? nf : 0.0f, ok ? ni : -INFINITY, &sb, &su, &sp);
    };
    gload(0);
    if (gwave) gscan(0);
    gload(L);
    // The block of C' is held as MFMA accumulators: wavefront w owns row
    // tiles w and w + 8 (16 rows each) and two quads of 64 columns; in a
    // quad, lane (l16, g) holds the four consecutive columns 4 l16 .. +3, one
    // in each of four MFMA tiles (tile x takes quad column 4n + x as its
    // column n), so that a lane's values of a row are one 16-byte group.
    // sacc[a][q][x][v] = C'[16 (w + 8a) + 4g + v][c0 + 64q + 4 l16 + x].
    // soff[a][q] is the byte offset of its row 4g in a [d_qk][d_v] record,
    // past every record when the tile lies outside the block.
    const int wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
    f32x4 sacc[2][2][4];
    unsigned soff[2][2];
    bool arow[2], aq[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        arow[x] = 16 * (wave + 8 * x) < dk;
        aq[x] = 64 * x < w;
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int q = 0; q < 2; ++q)
            soff[x][q] = (arow[x] && 64 * q + 4 * l16 < w)
                             ? (unsigned)(((16 * (wave + 8 * x) + 4 * g) * dv + c0 + 64 * q + 4 * l16) * 4)
                             : kFar;
    // n' (block 0, threads below d_qk) and m (thread d_qk) follow C' in the record
    const unsigned noff = (blk == 0 && tid <= dk) ? (unsigned)((dk * dv + tid) * 4) : kFar;
    {
        const __amdgpu_buffer_rsrc_t c0r =
            a.C0 ? rsrc(a.C0 + (size_t)p * dk * dv, (size_t)dk * dv * 4) : rsrc(a.ckpt, 0);
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const f32x4 y = buf_ld4(c0r, soff[x][q] + (unsigned)(v * dv * 4));
#pragma unroll
                    for (int e = 0; e < 4; ++e) sacc[x][q][e][v] = y[e];
                }
    }
    if (blk == 0)
        for (int e = tid; e < dk; e += NTS) ns[e] = a.n0 ? a.n0[(size_t)p * dk + e] : 0.0f;
    float m = a.m0 ? a.m0[p] : 0.0f;
    for (int c = 0; c < nch; ++c) {
        const int t0 = c * L;
        // this chunk's tiles and gates into LDS first: they wait only for the
        // loads issued a chunk ago, not for the record stores below (the
        // tiles of the last chunk are not used)
        kf.put(Ks, LK, dk, tid);
        vf.put(Vs, BVB, w, tid);
        if (gwave) {  // this chunk's gates: r = max(m, prefix max u)
            const float r = fmaxf(m, sp);
            const float r_last = __shfl(r, L - 1, 64);
            if (lane < L) wv[lane] = exp_e(su - r_last);
            if (lane == L - 1) {
                last[0] = sb;
                last[1] = r;
            }
        }
        // the state at this chunk's start (each thread reads and writes only
        // its own entries of ns; the other reads are discarded)
        const __amdgpu_buffer_rsrc_t rs = rsrc(base + (size_t)c * rec, rec * 4);
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                if (!arow[x] || !aq[q]) continue;  // uniform in the wavefront: the tile lies outside
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    buf_st4(f32x4{sacc[x][q][0][v], sacc[x][q][1][v], sacc[x][q][2][v], sacc[x][q][3][v]}, rs,
                            soff[x][q] + (unsigned)(v * dv * 4));
            }
        buf_st1(tid < dk ? ns[tid < dk ? tid : 0] : m, rs, noff);
        if (c + 1 == nch) break;  // the state after the last chunk is not needed
        fetch(t0 + L);
        lds_barrier();
        const float b_last = last[0], r_last = last[1];
        const float dec = exp_e(m - r_last);
        if (gwave) gscan(t0 + L);  // the next chunk's gates, off the chain
        gload(t0 + 2 * L);
        // C' <- dec C' + sum_j (w_j k_j) v_j^T on the matrix cores (k index = token)
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) sacc[x][q][e] *= dec;
#pragma unroll
        for (int s4 = 0; s4 < L / 4; ++s4) {
            const int j = 4 * s4 + g;
            const float wj = wv[j];
            f32x4 vb[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) vb[q] = ld4(&Vs[j * BVB + 64 * q + 4 * l16]);
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                if (!arow[x]) continue;  // uniform in the wavefront
                const float ka = wj * Ks[j * LK + 16 * (wave + 8 * x) + l16];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    if (!aq[q]) continue;
#pragma unroll
                    for (int e = 0; e < 4; ++e) sacc[x][q][e] = mfma4(ka, vb[q][e], sacc[x][q][e]);
                }
            }
        }
        if (blk == 0)
            for (int e = tid; e < dk; e += NTS) {
                float acc = dec * ns[e];
                for (int j = 0; j < L; ++j) acc = fmaf(wv[j], Ks[j * LK + e], acc);
                ns[e] = acc;
            }
        m = b_last + r_last;
        lds_barrier();  // the tiles are rewritten next chunk
    }
}

// Pass A: one workgroup per (chunk, pair).  P (the decayed causal q.k) and
// the denominators in float32 on the vector units; then on the matrix cores:
// the read-out num = sv (Q C') + P V by units of 64 value columns (C' rows
// read as 16-byte groups of four columns, one per MFMA tile, as in pass C's
// dv part), a and do~ from it in registers, and the a.v products of P~ as
// 2 x 2 tiles of [L][L], split over 16-column blocks across the wavefronts
// and summed through LDS.
template <typename IO>
__global__ __launch_bounds__(NTA) void bwd_a_kernel(BwdArgs a) {
    constexpr int LK = kBwdMaxDk + 4, LP = L + 1, NW = NTA / 64, NUM = kBwdMaxDv / 64;
    __shared__ __attribute__((aligned(16))) float Q[L * LK], K[L * LK];  // K's space later holds partial sums
    __shared__ float P[L * LP], part[L * NUM];
    __shared__ float gb[L], gu[L], gr[L], sv[L], fl[L], dd[L], den[L], beta[L], last[2];
    const int c = blockIdx.x, p = blockIdx.y, tid = threadIdx.x;
    const int dk = a.dk, dv = a.dv, T = a.T, t0 = c * L;
    const BwdLayout lay = bwd_layout(T, dk, dv);
    float *base = a.ckpt + (size_t)p * lay.total;
    const float *Cc = base + (size_t)c * lay.rec;  // C' rows of dv floats, then n', m
    const float *ncg = Cc + (size_t)dk * dv;
    const float m_prev = ncg[dk];
    float *Aw = base + lay.off_a + (size_t)c * L * dv;
    float *Pw = base + lay.off_p + (size_t)c * 2 * L * L;
    float *Sw = base + lay.off_s + (size_t)c * 4 * L;
    const size_t oqk = (size_t)p * T * dk, ov = (size_t)p * T * dv, og1 = (size_t)p * T;
    const size_t ioN = (size_t)T * dv * sizeof(IO);
    const __amdgpu_buffer_rsrc_t vr = rsrc(static_cast<const IO *>(a.v) + ov, ioN);
    const __amdgpu_buffer_rsrc_t orr = rsrc(static_cast<const IO *>(a.o) + ov, ioN);
    const __amdgpu_buffer_rsrc_t dhr = rsrc(static_cast<const IO *>(a.dh) + ov, ioN);

    load_tile(Q, LK, static_cast<const IO *>(a.q) + oqk, dk, t0, T, tid, NTA);
    load_tile(K, LK, static_cast<const IO *>(a.k) + oqk, dk, t0, T, tid, NTA);
    if (tid < 64) chunk_gates(a.ig + og1, a.fg + og1, t0, T, m_prev, gb, gu, gr, last);
    __syncthreads();
    const float r_last = last[1];
    if (tid < L) {
        sv[tid] = exp_e(m_prev - gr[tid]);
        fl[tid] = exp_e(-(gb[tid] + gr[tid]));
    }
    for (int e = tid; e < L * L; e += NTA) {
        const int i = e / L, j = e % L;
        float s = 0.0f;
        if (j <= i && t0 + i < T) s = dot(&Q[i * LK], &K[j * LK], dk) * exp_e(gu[j] - gr[i]);
        P[i * LP + j] = s;
    }
    __syncthreads();
    if (tid < L) {
        const int i = tid;
        float acc = 0.0f;
        for (int r = 0; r < dk; ++r) acc = fmaf(ncg[r], Q[i * LK + r], acc);
        acc *= sv[i];
        for (int j = 0; j <= i; ++j) acc += P[i * LP + j];
        dd[i] = acc;
        den[i] = fmaxf(fabsf(acc), fl[i]);
    }
    __syncthreads();

    const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    // ---- num, a, do~: value columns [b0, b0 + 64); x[tt][xx][v] holds token
    // 16 tt + 4g + v, column b0 + 4 l16 + xx
    const int NU = (dv + 63) / 64, NS = dk / 4;
    for (int bu = wave; bu < NU; bu += NW) {
        const int b0 = 64 * bu;
        const bool colok = b0 + 4 * l16 < dv;
        const __amdgpu_buffer_rsrc_t cr = rsrc(Cc, (size_t)dk * dv * 4);
        const __amdgpu_buffer_rsrc_t aw = rsrc(Aw, (size_t)L * dv * 4);
        const __amdgpu_buffer_rsrc_t gor = rsrc(a.go + ov, (size_t)T * dv * 4);
        const unsigned co = colok ? (unsigned)((g * dv + b0 + 4 * l16) * 4) : kFar;
        const unsigned rstep = (unsigned)(4 * dv * 4);
        f32x4 x[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int xx = 0; xx < 4; ++xx) x[tt][xx] = f32x4{0.f, 0.f, 0.f, 0.f};
        // sum_r q_i[r] C'[r][b]
        f32x4 ga[4], gb4[4];
        dv_gload(ga, cr, co, rstep, 0, NS);
        __builtin_amdgcn_sched_barrier(0);
        dv_gload(gb4, cr, co, rstep, 4, NS);
        __builtin_amdgcn_sched_barrier(0);
        for (int s0 = 0; s0 < NS; s0 += 8) {
            dv_gstep<LK>(x, ga, Q, l16, g, s0, 1.0f);
            dv_gload(ga, cr, co, rstep, s0 + 8, NS);
            __builtin_amdgcn_sched_barrier(0);
            dv_gstep<LK>(x, gb4, Q, l16, g, min(s0 + 4, NS - 4), s0 + 4 < NS ? 1.0f : 0.0f);
            dv_gload(gb4, cr, co, rstep, s0 + 12, NS);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float si = sv[16 * tt + 4 * g + v];
#pragma unroll
                for (int xx = 0; xx < 4; ++xx) x[tt][xx][v] *= si;
            }
        // + sum_{j <= i} P_ij v_j[b] (P zero above the diagonal; v zero past T)
#pragma unroll
        for (int s = 0; s < L / 4; ++s) {
            const int j = 4 * s + g;
            const f32x4 vb = Quad<IO>::cvt(
                Quad<IO>::load(vr, colok ? (unsigned)(((t0 + j) * dv + b0 + 4 * l16) * (int)sizeof(IO)) : kFar));
            const float p0 = P[l16 * LP + j], p1 = P[(16 + l16) * LP + j];
#pragma unroll
            for (int xx = 0; xx < 4; ++xx) {
                x[0][xx] = mfma4(p0, vb[xx], x[0][xx]);
                x[1][xx] = mfma4(p1, vb[xx], x[1][xx]);
            }
        }
        // a = dh sigmoid(o~) / den (to the workspace; zero past T, where dh
        // reads as zero), do~ (rows past T dropped), and a.num over these
        // columns per token
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = 16 * tt + 4 * g + v, t = t0 + i;
                const unsigned eo = colok ? (unsigned)((t * dv + b0 + 4 * l16) * (int)sizeof(IO)) : kFar;
                const f32x4 dh = Quad<IO>::cvt(Quad<IO>::load(dhr, eo));
                const f32x4 og = Quad<IO>::cvt(Quad<IO>::load(orr, eo));
                const float rd = 1.0f / den[i];
                f32x4 av, go;
                float an = 0.0f;
#pragma unroll
                for (int xx = 0; xx < 4; ++xx) {
                    const float sg = sigmoid(og[xx]), num = x[tt][xx][v];
                    av[xx] = dh[xx] * sg * rd;
                    go[xx] = dh[xx] * num * rd * sg * (1.0f - sg);
                    an = fmaf(av[xx], num, an);
                }
                buf_st4(go, gor, colok ? (unsigned)((t * dv + b0 + 4 * l16) * 4) : kFar);
                buf_st4(av, aw, colok ? (unsigned)((i * dv + b0 + 4 * l16) * 4) : kFar);
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) an += __shfl_xor(an, o, 64);
                if (l16 == 0) part[i * NUM + bu] = an;
            }
    }
    __syncthreads();  // a rows in the workspace and the row partials visible
    if (tid < L) {
        const int i = tid;
        float an = 0.0f;
        for (int b = 0; b < NU; ++b) an += part[i * NUM + b];
        beta[i] = fabsf(dd[i]) > fl[i] ? (dd[i] > 0.0f ? -an : an) / den[i] : 0.0f;
        Sw[i] = sv[i];
        Sw[L + i] = exp_e(gu[i] - r_last);
        Sw[2 * L + i] = beta[i];
        if (i == 0) Sw[3 * L] = exp_e(m_prev - r_last);
    }
    // ---- a.v for P~: tile (ti, tj) of [L][L]; this wavefront takes the
    // 16-column blocks wave, wave + 8, ... (up to four; blocks past d_v load
    // zeros).  pt[ti][tj][v] = sum over its blocks of a_i . v_j, i = 16 ti +
    // 4g + v, j = 16 tj + l16.
    {
        const int NB16 = dv / 16;
        const __amdgpu_buffer_rsrc_t ar = rsrc(Aw, (size_t)L * dv * 4);
        f32x4 a4[4][2];
        typename Quad<IO>::raw v4[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kb = wave + NW * u;
            const bool ok = kb < NB16;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                a4[u][h] = buf_ld4(ar, ok ? (unsigned)(((16 * h + l16) * dv + 16 * kb + 4 * g) * 4) : kFar);
                v4[u][h] = Quad<IO>::load(
                    vr, ok ? (unsigned)(((t0 + 16 * h + l16) * dv + 16 * kb + 4 * g) * (int)sizeof(IO)) : kFar);
            }
        }
        f32x4 pt[2][2];
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int tj = 0; tj < 2; ++tj) pt[ti][tj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x4 vb0 = Quad<IO>::cvt(v4[u][0]), vb1 = Quad<IO>::cvt(v4[u][1]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int ti = 0; ti < 2; ++ti) {
                    pt[ti][0] = mfma4(a4[u][ti][s], vb0[s], pt[ti][0]);
                    pt[ti][1] = mfma4(a4[u][ti][s], vb1[s], pt[ti][1]);
                }
        }
        float *red = K;  // [NW][L][L] partial sums (K is no longer read)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int tj = 0; tj < 2; ++tj)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    red[(wave * L + 16 * ti + 4 * g + v) * L + 16 * tj + l16] = pt[ti][tj][v];
    }
    __syncthreads();
    // P~_ij = (a_i.v_j + beta_i) e^{u_j - r_i}, and P, to the workspace
    for (int e = tid; e < L * L; e += NTA) {
        const int i = e / L, j = e % L;
        float pa = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) pa += K[w2 * L * L + e];
        Pw[e] = P[i * LP + j];
        Pw[L * L + e] = (j <= i && t0 + i < T) ? (pa + beta[i]) * exp_e(gu[j] - gr[i]) : 0.0f;
    }
}

// Pass B: one workgroup per (block of BVB value columns, pair): G* and g*
// backwards over the chunks, G*'s [d_qk][BVB] block in registers (as MFMA
// accumulators, laid out as in the checkpoint pass); block 0 also carries g*.
template <typename IO>
__global__ __launch_bounds__(NTS) void bwd_b_kernel(BwdArgs a) {
    constexpr int LK = kBwdMaxDk + 4;
    __shared__ __attribute__((aligned(16))) float Qs[L * LK + 4], As[L * BVB + 4];
    __shared__ float gs[kBwdMaxDk], sq[L], sqb[L], dcv[L], red[NTS];
    const int blk = blockIdx.x, p = blockIdx.y, tid = threadIdx.x;
    const int dk = a.dk, dv = a.dv, T = a.T;
    const int c0 = blk * BVB, w = min(BVB, dv - c0);  // this block's columns [c0, c0 + w)
    const BwdLayout lay = bwd_layout(T, dk, dv);
    const int nch = (int)lay.nch;
    float *base = a.ckpt + (size_t)p * lay.total;
    const IO *qg = static_cast<const IO *>(a.q) + (size_t)p * T * dk;
    const __amdgpu_buffer_rsrc_t qr = rsrc(qg, (size_t)T * dk * sizeof(IO));
    // the next chunk's Q tile, a rows and scalars load while the current
    // chunk computes; lane l of every wavefront takes token l's sv and beta
    // and slot l of the chunk's decay row (only slot 0 holds the decay; the
    // others are unused workspace)
    TileFetch<IO, L * kBwdMaxDk / 4 / NTS, NTS> qf;
    TileFetch<float, L * BVB / 4 / NTS, NTS> af;
    const int l = tid & (L - 1);
    float s_sv, s_beta, s_dec;
    auto fetch = [&](int c) {
        const float *Sw = base + lay.off_s + (size_t)c * 4 * L;
        qf.fetch(qr, dk, 0, dk, c * L, tid);
        af.fetch(rsrc(base + lay.off_a + (size_t)c * L * dv, (size_t)L * dv * 4), dv, c0, w, 0, tid);
        s_sv = Sw[l];
        s_beta = Sw[2 * L + l];
        s_dec = Sw[3 * L + l];
    };
    fetch(nch - 1);
    // G*'s block as MFMA accumulators, laid out as C' in the checkpoint pass:
    // gacc[a][q][x][v] = G*[16 (w + 8a) + 4g + v][c0 + 64q + 4 l16 + x]
    const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    f32x4 gacc[2][2][4];
    unsigned soff[2][2];
    bool arow[2], aq[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        arow[x] = 16 * (wave + 8 * x) < dk;
        aq[x] = 64 * x < w;
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            soff[x][q] = (arow[x] && 64 * q + 4 * l16 < w)
                             ? (unsigned)(((16 * (wave + 8 * x) + 4 * g) * dv + c0 + 64 * q + 4 * l16) * 4)
                             : kFar;
#pragma unroll
            for (int e = 0; e < 4; ++e) gacc[x][q][e] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    const unsigned goff = (blk == 0 && tid < dk) ? (unsigned)((dk * dv + tid) * 4) : kFar;  // g*
    for (int e = tid; e < dk; e += NTS) gs[e] = 0.0f;
    for (int c = nch - 1; c >= 0; --c) {
        // this chunk's tiles and scalars into LDS first: they wait only for
        // the loads issued a chunk ago, not for the record stores below
        qf.put(Qs, LK, dk, tid);
        af.put(As, BVB, w, tid);
        sq[l] = s_sv;             // sv_i
        sqb[l] = s_sv * s_beta;   // sv_i beta_i
        dcv[l] = s_dec;
        // the carried gradients entering chunk c (each thread reads and
        // writes only its own entries of gs; the other reads are discarded)
        const __amdgpu_buffer_rsrc_t gsd = rsrc(base + lay.off_g + (size_t)c * lay.grec, lay.grec * 4);
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                if (!arow[x] || !aq[q]) continue;  // uniform in the wavefront: the tile lies outside
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    buf_st4(f32x4{gacc[x][q][0][v], gacc[x][q][1][v], gacc[x][q][2][v], gacc[x][q][3][v]}, gsd,
                            soff[x][q] + (unsigned)(v * dv * 4));
            }
        buf_st1(gs[tid < dk ? tid : 0], gsd, goff);
        fetch(max(c - 1, 0));
        lds_barrier();
        const float dec = dcv[0];
        // G* <- dec G* + sum_i (sv_i q_i) a_i^T on the matrix cores (k index = token)
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) gacc[x][q][e] *= dec;
#pragma unroll
        for (int s4 = 0; s4 < L / 4; ++s4) {
            const int i = 4 * s4 + g;
            const float si = sq[i];
            f32x4 ab[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) ab[q] = ld4(&As[i * BVB + 64 * q + 4 * l16]);
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                if (!arow[x]) continue;  // uniform in the wavefront
                const float qa = si * Qs[i * LK + 16 * (wave + 8 * x) + l16];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    if (!aq[q]) continue;
#pragma unroll
                    for (int e = 0; e < 4; ++e) gacc[x][q][e] = mfma4(qa, ab[q][e], gacc[x][q][e]);
                }
            }
        }
        if (blk == 0)
            for (int e = tid; e < dk; e += NTS) {
                float acc = dec * gs[e];
                for (int i = 0; i < L; ++i) acc = fmaf(sqb[i], Qs[i * LK + e], acc);
                gs[e] = acc;
            }
        lds_barrier();  // the tiles are rewritten next chunk
    }
    // G*, g* after the first chunk: the initial state's gradients, and this
    // block's part of <dC0, C0>
    float part = 0.0f;
    {
        const size_t pb = (size_t)p * dk * dv, nb = (size_t)dk * dv * 4;
        const __amdgpu_buffer_rsrc_t c0r = a.C0 ? rsrc(a.C0 + pb, nb) : rsrc(a.ckpt, 0);
        const __amdgpu_buffer_rsrc_t g0r = a.gC0 ? rsrc(a.gC0 + pb, nb) : rsrc(a.ckpt, 0);
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const unsigned off = soff[x][q] + (unsigned)(v * dv * 4);
                    const f32x4 gv{gacc[x][q][0][v], gacc[x][q][1][v], gacc[x][q][2][v], gacc[x][q][3][v]};
                    buf_st4(gv, g0r, off);
                    const f32x4 cv = buf_ld4(c0r, off);
#pragma unroll
                    for (int y = 0; y < 4; ++y) part = fmaf(gv[y], cv[y], part);
                }
    }
    if (blk == 0 && a.gn0)
        for (int e = tid; e < dk; e += NTS) a.gn0[(size_t)p * dk + e] = gs[e];
    red[tid] = part;
    __syncthreads();
    for (int s2 = NTS / 2; s2 > 0; s2 >>= 1) {
        if (tid < s2) red[tid] += red[tid + s2];
        __syncthreads();
    }
    if (tid == 0) base[lay.off_m + blk] = red[0];
}

// Pass C: one workgroup per (chunk, pair); its contractions run on the
// matrix cores in float32 (16 x 16 output tiles, one per wavefront at a time).
//   dq, dk by 16 rows of d_qk: C' a and G* v contract over the value columns,
//     which each lane reads four at a time straight from the records (the
//     k index of successive MFMAs is permuted alike in both operands), then
//     are scaled per token, and the in-chunk P~ K and P~^T Q are added
//     through the same accumulators;
//   dv by 64 value columns: G*^T k over the rows of G* (a lane reads four
//     consecutive columns of a row, one for each of four MFMA tiles), scaled
//     per token, plus P^T a.
// q.dq and k.dk are summed per (token, 16 rows) into partials for the gates.
template <typename IO>
__global__ __launch_bounds__(NTA) void bwd_c_kernel(BwdArgs a) {
    constexpr int LK = kBwdMaxDk + 4, LP = L + 1, NRTM = kBwdMaxDk / 16, NW = NTA / 64;
    __shared__ __attribute__((aligned(16))) float Q[L * LK], K[L * LK];
    __shared__ float P[L * LP], PT[L * LP], sv[L], wv[L], beta[L];
    __shared__ float pq[L * NRTM], pk[L * NRTM];
    const int c = blockIdx.x, p = blockIdx.y, tid = threadIdx.x;
    const int dk = a.dk, dv = a.dv, T = a.T, t0 = c * L;
    const BwdLayout lay = bwd_layout(T, dk, dv);
    float *base = a.ckpt + (size_t)p * lay.total;
    const float *Cc = base + (size_t)c * lay.rec;
    const float *ncg = Cc + (size_t)dk * dv;
    const float *Aw = base + lay.off_a + (size_t)c * L * dv;
    const float *Pw = base + lay.off_p + (size_t)c * 2 * L * L;
    const float *Sw = base + lay.off_s + (size_t)c * 4 * L;
    const float *Gw = base + lay.off_g + (size_t)c * lay.grec;  // G* entering chunk c, then g*
    const size_t oqk = (size_t)p * T * dk, ov = (size_t)p * T * dv, og1 = (size_t)p * T;

    load_tile(Q, LK, static_cast<const IO *>(a.q) + oqk, dk, t0, T, tid, NTA);
    load_tile(K, LK, static_cast<const IO *>(a.k) + oqk, dk, t0, T, tid, NTA);
    for (int e = tid; e < L * L; e += NTA) {
        P[(e / L) * LP + e % L] = Pw[e];
        PT[(e / L) * LP + e % L] = Pw[L * L + e];
    }
    if (tid < L) {
        sv[tid] = Sw[tid];
        wv[tid] = Sw[L + tid];
        beta[tid] = Sw[2 * L + tid];
    }
    __syncthreads();

    const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const __amdgpu_buffer_rsrc_t vr = rsrc(static_cast<const IO *>(a.v) + ov, (size_t)T * dv * sizeof(IO));
    // outputs through descriptors ending at token T: rows past it are dropped
    const __amdgpu_buffer_rsrc_t oq = rsrc(a.gq + oqk, (size_t)T * dk * 4);
    const __amdgpu_buffer_rsrc_t ok_ = rsrc(a.gk + oqk, (size_t)T * dk * 4);
    const __amdgpu_buffer_rsrc_t ovr = rsrc(a.gv + ov, (size_t)T * dv * 4);

    // ---- dq and dk: rows [r0, r0 + 16) of d_qk for all L tokens
    const int NRT = dk / 16;
    for (int rt = wave; rt < NRT; rt += NW) {
        const int r0 = 16 * rt;
        f32x4 xq[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, xk[2] = {xq[0], xq[0]};
        // lane (l16, g) reads C'[r0 + l16][b0 + 4g .. +3] and G* likewise, and
        // a_i, v_i of tokens i = l16 and 16 + l16 at the same columns, all
        // through buffer loads (the compiler keeps those where they are
        // issued, a block pair ahead of their use; it moved plain loads down
        // to their uses)
        const __amdgpu_buffer_rsrc_t cr = rsrc(Cc, (size_t)dk * dv * 4), grs = rsrc(Gw, (size_t)dk * dv * 4);
        const __amdgpu_buffer_rsrc_t ar = rsrc(Aw, (size_t)L * dv * 4);
        const unsigned so = (unsigned)(((r0 + l16) * dv + 4 * g) * 4), ao = (unsigned)((l16 * dv + 4 * g) * 4);
        const unsigned astep = (unsigned)(16 * dv * 4);
        const unsigned vo = (unsigned)(((t0 + l16) * dv + 4 * g) * (int)sizeof(IO));
        const unsigned vstep = (unsigned)(16 * dv * (int)sizeof(IO));
        // (v stays in its I/O type until used: a conversion before the
        // scheduling barrier below would wait for the load)
        struct Blk { f32x4 c, g, a0, a1; typename Quad<IO>::raw v0, v1; };
        auto fetch = [&](int b0) {
            Blk x;
            const unsigned fb = (unsigned)(b0 * 4), eb = (unsigned)(b0 * (int)sizeof(IO));
            x.c = buf_ld4(cr, so + fb);
            x.g = buf_ld4(grs, so + fb);
            x.a0 = buf_ld4(ar, ao + fb);
            x.a1 = buf_ld4(ar, ao + astep + fb);
            x.v0 = Quad<IO>::load(vr, vo + eb);
            x.v1 = Quad<IO>::load(vr, vo + vstep + eb);
            return x;
        };
        auto step = [&](const Blk &x, float on) {
            const f32x4 v0 = Quad<IO>::cvt(x.v0), v1 = Quad<IO>::cvt(x.v1);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                xq[0] = mfma4(on * x.a0[s], x.c[s], xq[0]);
                xq[1] = mfma4(on * x.a1[s], x.c[s], xq[1]);
                xk[0] = mfma4(on * v0[s], x.g[s], xk[0]);
                xk[1] = mfma4(on * v1[s], x.g[s], xk[1]);
            }
        };
        // blocks of 16 value columns alternate between two register sets, each
        // reloaded right after its MFMAs are issued (so the other set's MFMAs
        // cover its loads, and no loop-carried copy waits for a load); an odd
        // last block reads a valid block again and is multiplied by zero
        const int last = dv - 16;
        Blk xa = fetch(0);
        __builtin_amdgcn_sched_barrier(0);  // all of set A's loads before set B's
        Blk xb = fetch(min(16, last));
        __builtin_amdgcn_sched_barrier(0);
        for (int b0 = 0; b0 < dv; b0 += 32) {
            step(xa, 1.0f);
            xa = fetch(min(b0 + 32, last));
            __builtin_amdgcn_sched_barrier(0);
            step(xb, b0 + 16 < dv ? 1.0f : 0.0f);
            xb = fetch(min(b0 + 48, last));
            __builtin_amdgcn_sched_barrier(0);
        }
        // scale per token: dq_i = sv_i (C' a_i + n' beta_i), dk_i = w_i (G* v_i + g*)
        const float nr = ncg[r0 + l16], gr_ = Gw[(size_t)dk * dv + r0 + l16];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = 16 * tt + 4 * g + v;
                xq[tt][v] = sv[i] * fmaf(nr, beta[i], xq[tt][v]);
                xk[tt][v] = wv[i] * (xk[tt][v] + gr_);
            }
        // + sum_j P~_ij k_j and + sum_i2 P~_i2,i q_i2 (zero outside j <= i)
#pragma unroll
        for (int s = 0; s < L / 4; ++s) {
            const int j = 4 * s + g;
            const float kb = K[j * LK + r0 + l16], qb = Q[j * LK + r0 + l16];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                xq[tt] = mfma4(PT[(16 * tt + l16) * LP + j], kb, xq[tt]);
                xk[tt] = mfma4(PT[j * LP + 16 * tt + l16], qb, xk[tt]);
            }
        }
        // outputs, and q.dq, k.dk over these 16 rows per token
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = 16 * tt + 4 * g + v, r = r0 + l16;
                const unsigned off = (unsigned)(((t0 + i) * dk + r) * 4);
                buf_st1(xq[tt][v], oq, off);
                buf_st1(xk[tt][v], ok_, off);
                float sq = Q[i * LK + r] * xq[tt][v], sk = K[i * LK + r] * xk[tt][v];
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) {
                    sq += __shfl_xor(sq, o, 64);
                    sk += __shfl_xor(sk, o, 64);
                }
                if (l16 == 0) {
                    pq[i * NRTM + rt] = sq;
                    pk[i * NRTM + rt] = sk;
                }
            }
    }

    // ---- dv: value columns [b0, b0 + 64) for all L tokens.  Lane (l16, g)
    // reads four consecutive columns b0 + 4 l16 .. +3 of a row of G* (or of
    // a), one for each of four MFMA tiles: tile x takes column b0 + 4n + x as
    // its column n, so each lane's outputs of a token are again four
    // consecutive columns.  Lanes past d_v load zeros and store nothing.  The
    // wavefronts take these units in reverse order, so that those without
    // d_qk rows start first.
    const int NBU = (dv + 63) / 64, NS = dk / 4;  // NS: steps of 4 rows of G*, a multiple of 4
    for (int bu = NW - 1 - wave; bu < NBU; bu += NW) {
        const int b0 = 64 * bu;
        const __amdgpu_buffer_rsrc_t gsr = rsrc(Gw, (size_t)dk * dv * 4), asr = rsrc(Aw, (size_t)L * dv * 4);
        const bool colok = b0 + 4 * l16 < dv;
        const unsigned go = colok ? (unsigned)((g * dv + b0 + 4 * l16) * 4) : kFar;
        const unsigned rstep = (unsigned)(4 * dv * 4);  // four rows
        f32x4 x[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int xx = 0; xx < 4; ++xx) x[tt][xx] = f32x4{0.f, 0.f, 0.f, 0.f};
        // w_j sum_r k_j[r] G*[r][b] over steps s (rows 4s + g), in groups of
        // four steps alternating between two register sets, each reloaded
        // right after use; a group past the last one reloads a valid group
        // and its K operand is zero
        f32x4 ga[4], gb[4];
        dv_gload(ga, gsr, go, rstep, 0, NS);
        __builtin_amdgcn_sched_barrier(0);
        dv_gload(gb, gsr, go, rstep, 4, NS);
        __builtin_amdgcn_sched_barrier(0);
        for (int s0 = 0; s0 < NS; s0 += 8) {
            dv_gstep<LK>(x, ga, K, l16, g, s0, 1.0f);
            dv_gload(ga, gsr, go, rstep, s0 + 8, NS);
            __builtin_amdgcn_sched_barrier(0);
            dv_gstep<LK>(x, gb, K, l16, g, min(s0 + 4, NS - 4), s0 + 4 < NS ? 1.0f : 0.0f);
            dv_gload(gb, gsr, go, rstep, s0 + 12, NS);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float wj = wv[16 * tt + 4 * g + v];
#pragma unroll
                for (int xx = 0; xx < 4; ++xx) x[tt][xx][v] *= wj;
            }
        // + sum_{i >= j} P_ij a_i[b]  (steps over tokens i = 4s + g)
        const unsigned ao2 = colok ? (unsigned)((g * dv + b0 + 4 * l16) * 4) : kFar;
#pragma unroll
        for (int s = 0; s < L / 4; ++s) {
            const f32x4 av = buf_ld4(asr, ao2 + (unsigned)s * rstep);
            const int i = 4 * s + g;
            const float p0 = P[i * LP + l16], p1 = P[i * LP + 16 + l16];
#pragma unroll
            for (int xx = 0; xx < 4; ++xx) {
                x[0][xx] = mfma4(p0, av[xx], x[0][xx]);
                x[1][xx] = mfma4(p1, av[xx], x[1][xx]);
            }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + 16 * tt + 4 * g + v;
                buf_st4(f32x4{x[tt][0][v], x[tt][1][v], x[tt][2][v], x[tt][3][v]}, ovr,
                        colok ? (unsigned)((t * dv + b0 + 4 * l16) * 4) : kFar);
            }
    }
    __syncthreads();  // the row partials of q.dq and k.dk complete
    // gate gradients: di = k.dk; the in-chunk part of df (reverse cumsum of
    // q.dq - k.dk) and the chunk's total, for the carry of pass D
    if (tid < 64) {
        const int j = tid, t = t0 + j;
        const bool ok = j < L && t < T;
        float di = 0.0f, x = 0.0f;
        if (ok) {
            float sq = 0.0f;
            for (int r = 0; r < NRT; ++r) {
                di += pk[j * NRTM + r];
                sq += pq[j * NRTM + r];
            }
            x = sq - di;
        }
        float y = x;  // sum over lanes >= j
        for (int o = 1; o < 64; o <<= 1) {
            const float z = __shfl_down(y, o, 64);
            if (j + o < 64) y += z;
        }
        if (ok) {
            a.gi[og1 + t] = di;
            a.gf[og1 + t] = y;
        }
        if (j == 0) base[lay.off_x + c] = y;
    }
}

// Pass D: one wavefront per pair: df~'s carry from the later chunks, and dm0.
__global__ __launch_bounds__(64) void bwd_d_kernel(BwdArgs a) {
    const int p = blockIdx.x, lane = threadIdx.x;
    const int dk = a.dk, dv = a.dv, T = a.T;
    const BwdLayout lay = bwd_layout(T, dk, dv);
    const int nch = (int)lay.nch;
    const float *base = a.ckpt + (size_t)p * lay.total;
    const size_t og1 = (size_t)p * T;
    // groups of 64 chunks from the end: lane j takes chunk c0 + j; its carry
    // is the sum of the totals of every later chunk (an exclusive suffix sum,
    // within the group by a wavefront scan, plus the later groups' running
    // sum), which it then adds to the df~ of its chunk's tokens
    float running = 0.0f;
    for (int c0 = (nch - 1) / 64 * 64; c0 >= 0; c0 -= 64) {
        const int c = c0 + lane;
        const float x = c < nch ? base[lay.off_x + c] : 0.0f;
        float y = x;  // sum over lanes >= this one
        for (int o = 1; o < 64; o <<= 1) {
            const float z = __shfl_down(y, o, 64);
            if (lane + o < 64) y += z;
        }
        const float carry = running + (y - x);
        running += __shfl(y, 0, 64);
        if (c < nch) {
            float *gf = a.gf + og1 + (size_t)c * L;
            const int n = min(L, T - c * L);
            for (int i = 0; i < n; ++i) gf[i] += carry;
        }
    }
    if (a.gm0) {
        float part = 0.0f;
        if (a.n0)
            for (int e = lane; e < dk; e += 64) part = fmaf(a.gn0[(size_t)p * dk + e], a.n0[(size_t)p * dk + e], part);
        for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
        if (lane == 0) {
            float s = part;
            const int nb = (dv + BVB - 1) / BVB;
            for (int b = 0; b < nb; ++b) s += base[lay.off_m + b];
            a.gm0[p] = s;
        }
    }
}

template <typename IO>
hipError_t launch_passes(const BwdArgs &a, hipStream_t s) {
    const int nch = (a.T + L - 1) / L, nb = (a.dv + BVB - 1) / BVB;
    hipLaunchKernelGGL(bwd_ckpt_kernel<IO>, dim3(nb, a.BH), dim3(NTS), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_a_kernel<IO>, dim3(nch, a.BH), dim3(NTA), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_b_kernel<IO>, dim3(nb, a.BH), dim3(NTS), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_c_kernel<IO>, dim3(nch, a.BH), dim3(NTA), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_d_kernel, dim3(a.BH), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, int io_bf16, hipStream_t s) {
    return io_bf16 ? launch_passes<bf16>(a, s) : launch_passes<float>(a, s);
}

}  // namespace mlstm
