// prefill_bf16.hpp -- chunkwise mLSTM forward for bf16 I/O on gfx950.
//
// Same mathematics as prefill_kernel.hpp (the chunkwise form of the xLSTM
// note's mLSTM recurrence, "mLSTM (matrix LSTM)" section, with the
// stabilizer of its "sLSTM" section): per chunk of L tokens, with
// b = in-chunk cumsum of f~, u_j = i~_j - b_j, r_i = max(m, max_{j<=i} u_j),
//   h_i = sigmoid(o~_i) (sum_j P_ij v_j + e^{m-r_i} C'^T q_i)
//                       / max(|sum_j P_ij + e^{m-r_i} n'.q_i|, e^{-(b_i+r_i)}),
//   P_ij = (q_i.k_j) e^{u_j - r_i} (j <= i),
//   C' <- e^{m-r_L} C' + sum_j e^{u_j-r_L} k_j v_j^T, n' likewise, m <- b_L + r_L.
//
// This is the bf16 schedule built around two gfx950 features:
//  * global -> LDS copies (global_load_lds, 16 bytes per lane) stage Q, K and
//    V without passing through registers; K and V are double buffered (the
//    next chunk streams in during the whole current chunk), Q is reloaded
//    once the current chunk's d_qk loop is done with it;
//  * the LDS transpose read (ds_read_b64_tr_b16) produces MFMA fragments of
//    K^T and V^T (token index along k) straight from the row-major tiles, so
//    nothing is ever written transposed.
// Tiles are row-major with 16-byte granules XOR-swizzled per row (granule
// g of row r lives at g ^ swz(r)), which keeps the 16-row fragment reads,
// the transpose reads and the copies free of bank conflicts.
//
// Work split: one workgroup = one (pair, segment, BV value columns); 4
// wavefronts, each owning BV/4 columns of the d_qk x BV state C' in
// registers (float32, MFMA accumulator layout).  Per chunk:
//   O^T  = C'^T Q^T        C' split into bf16 high + bf16 remainder (2 MFMAs),
//                          so the carried state keeps ~16 bits in the read-out
//   S^T  = K Q^T           causal 16x16 tiles spread over the wavefronts
//   qn   = Q n'            (one 16-token tile per wavefront, n' split too)
//   P    = S (x) decay     -> LDS (bf16);  O^T += V^T P^T;  h written
//   C'   = decay C' + K^T (w (x) V),  n' = decay n' + K^T w  (w split)
// The chunk's gate quantities are computed one chunk ahead by wavefront 0
// into a double-buffered table, so a chunk needs two workgroup barriers.
#pragma once

#include "prefill_kernel.hpp"

namespace mlstm {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int L_, int DKP_, int BV_>
struct Bf16Cfg {
    static constexpr int L = L_, DKP = DKP_, BV = BV_, NW = 4, NTH = 256;
    static constexpr int LP = L < 32 ? 32 : L;       // token rows held (k of 32 for the MFMA)
    static constexpr int NT = L / 16, NCT = NT * (NT + 1) / 2, MYT = (NCT + NW - 1) / NW;
    static constexpr int NAT = DKP / 16, NKS = DKP / 32, NJS = LP / 32;
    static constexpr int WC = BV / NW, NBT = WC / 16;
    static constexpr int QG = DKP / 8;                // 16-byte granules per Q/K row
    static constexpr int VG = BV / 8;                 // granules per V row
    static constexpr int PG = LP / 8;                 // granules per P row
    static constexpr int NA_W = NAT / NW;             // n' tiles per wavefront
    static constexpr size_t LDS_BYTES =
        2 * ((size_t)LP * DKP + 2 * (size_t)LP * DKP + 2 * (size_t)LP * BV + (size_t)L * LP) +
        4 * (2 * (5 * (size_t)LP + 4) + NCT * 16 + L + DKP);
    static_assert(NBT >= 1 && WC % 16 == 0, "whole 16-column tiles per wavefront");
    static_assert(NAT % NW == 0, "n' tiles spread evenly");
    static_assert(L <= 64, "one token per lane in the gate scan");
};

// granule swizzle: within each aligned group of 8 granules of a row
template <int GPR>
__device__ __forceinline__ int swz(int row) {
    constexpr int m = GPR < 8 ? GPR - 1 : 7;
    return (((row & 3) << 1) | ((row >> 2) & 1)) & m;
}
// element offset of (row, col) in a swizzled row-major bf16 tile with GPR granules per row
template <int GPR>
__device__ __forceinline__ int sw_off(int row, int col) {
    return row * GPR * 8 + ((((col >> 3) ^ swz<GPR>(row))) << 3) + (col & 7);
}

__device__ __forceinline__ bf16x4 tr_read(const bf16 *p) {
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    return __builtin_bit_cast(bf16x4, r);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// split 8 floats into bf16 high parts and bf16 remainders
__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16 h = (bf16)x[e];
        hi[e] = h;
        lo[e] = (bf16)(x[e] - (float)h);
    }
}

template <int L, int DKP, int BV, bool STATE_ONLY>
__global__ __launch_bounds__(256, 1) void mlstm_bf16_kernel(FwdArgs a) {
    using Cfg = Bf16Cfg<L, DKP, BV>;
    constexpr int NW = Cfg::NW, NTH = Cfg::NTH, LP = Cfg::LP, NT = Cfg::NT, NCT = Cfg::NCT;
    constexpr int MYT = Cfg::MYT, NAT = Cfg::NAT, NKS = Cfg::NKS, NJS = Cfg::NJS, WC = Cfg::WC;
    constexpr int NBT = Cfg::NBT, QG = Cfg::QG, VG = Cfg::VG, PG = Cfg::PG, NA_W = Cfg::NA_W;

    __shared__ __attribute__((aligned(16))) bf16 Qs[LP * DKP];
    __shared__ __attribute__((aligned(16))) bf16 Ks[2][LP * DKP];
    __shared__ __attribute__((aligned(16))) bf16 Vs[2][LP * BV];
    __shared__ __attribute__((aligned(16))) bf16 Ps[L * LP];
    // gate tables, double buffered: u, r, s, floor, w [LP] and 4 scalars
    __shared__ __attribute__((aligned(16))) float gt[2][5 * LP + 4];
    __shared__ float den_part[NCT * 16];
    __shared__ float qn[L];
    __shared__ __attribute__((aligned(16))) float nsh[DKP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;

    const int nwg = gridDim.x;
    int logical = blockIdx.x;
    if ((nwg & 7) == 0) logical = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int gseg = STATE_ONLY ? a.nseg - 1 : a.nseg;
    const int tile = logical % a.ntile;
    const int rest = logical / a.ntile;
    const int seg = rest % gseg;
    const int bh = rest / gseg;

    const int dk = a.dk, dv = a.dv, T = a.T;
    const int t_begin = seg * a.seg_len;
    const int t_end = min(t_begin + a.seg_len, T);
    const int nchunks = (t_end - t_begin + L - 1) / L;
    const int col0 = tile * BV;
    const int wcol0 = wave * WC;
    const int bv_here = min(BV, dv - col0);

    const bf16 *qg = static_cast<const bf16 *>(a.q) + (size_t)bh * T * dk;
    const bf16 *kg = static_cast<const bf16 *>(a.k) + (size_t)bh * T * dk;
    const bf16 *vg = static_cast<const bf16 *>(a.v) + (size_t)bh * T * dv;
    const bf16 *og = static_cast<const bf16 *>(a.o) + (size_t)bh * T * dv;
    bf16 *hg = static_cast<bf16 *>(a.h) + (size_t)bh * T * dv;
    const float *igg = a.ig + (size_t)bh * T;
    const float *fgg = a.fg + (size_t)bh * T;

    // ---- zero all tiles once (padding columns/rows and P's upper tiles stay zero)
    {
        uint4 *p;
        p = reinterpret_cast<uint4 *>(Qs);
        for (int e = tid; e < LP * DKP / 8; e += NTH) p[e] = make_uint4(0, 0, 0, 0);
        p = reinterpret_cast<uint4 *>(&Ks[0][0]);
        for (int e = tid; e < 2 * LP * DKP / 8; e += NTH) p[e] = make_uint4(0, 0, 0, 0);
        p = reinterpret_cast<uint4 *>(&Vs[0][0]);
        for (int e = tid; e < 2 * LP * BV / 8; e += NTH) p[e] = make_uint4(0, 0, 0, 0);
        p = reinterpret_cast<uint4 *>(Ps);
        for (int e = tid; e < L * LP / 8; e += NTH) p[e] = make_uint4(0, 0, 0, 0);
        for (int e = tid; e < 2 * (5 * LP + 4); e += NTH) (&gt[0][0])[e] = 0.0f;
    }

    // ---- initial state
    const size_t rec = seg_state_floats(dk, dv);
    const float *Cs = nullptr, *ns = nullptr;
    float m_prev = 0.0f;
    if (STATE_ONLY) {
        m_prev = -1e30f;
    } else if (a.seg_in) {
        const float *r = a.seg_in + ((size_t)bh * a.nseg + seg) * rec;
        Cs = r;
        ns = r + (size_t)dk * dv;
        m_prev = r[(size_t)dk * dv + dk];
    } else if (a.C0) {
        Cs = a.C0 + (size_t)bh * dk * dv;
        ns = a.n0 + (size_t)bh * dk;
        m_prev = a.m0[bh];
    }
    f32x4 Cr[NAT][NBT];
#pragma unroll
    for (int at = 0; at < NAT; ++at)
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt) {
            const int b = col0 + wcol0 + 16 * bt + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * at + 4 * g4 + r;
                Cr[at][bt][r] = (Cs && row < dk && b < dv) ? Cs[(size_t)row * dv + b] : 0.0f;
            }
        }
    // n' tiles owned by this wavefront (a-tiles wave*NA_W ...), MFMA layout, column 0
    f32x4 Nr[NA_W];
#pragma unroll
    for (int x = 0; x < NA_W; ++x) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * (wave * NA_W + x) + 4 * g4 + r;
            Nr[x][r] = (ns && l16 == 0 && row < dk) ? ns[row] : 0.0f;
        }
    }
    for (int e = tid; e < DKP; e += NTH) nsh[e] = (ns && e < dk) ? ns[e] : 0.0f;

    // ---- global -> LDS copies (16 bytes per lane, 64 consecutive granules per instruction)
    // Physical granule p of a tile -> (row, logical granule); the lane fetches
    // the logical granule so that the LDS image is the swizzled layout.
    auto copy_tile = [&](bf16 *dst, const bf16 *src, int ld, int gpr_log2, int cols_valid_g,
                         int rows, int tc) {
        const int total = rows << gpr_log2;     // granules in the tile
        const int gpr = 1 << gpr_log2;
        for (int blk = wave * 64; blk < total; blk += NW * 64) {
            const int p = blk + lane;
            const int row = p >> gpr_log2;
            const int pg = p & (gpr - 1);
            const int m = (gpr < 8 ? gpr - 1 : 7);
            const int gl = pg ^ ((((row & 3) << 1) | ((row >> 2) & 1)) & m);
            const int t = min(tc + row, t_end - 1);
            if (gl < cols_valid_g)
                __builtin_amdgcn_global_load_lds(
                    (const void *)(src + (size_t)t * ld + gl * 8),
                    (lds_void *)(dst + blk * 8), 16, 0, 0);
        }
    };
    constexpr int QGL = QG == 4 ? 2 : QG == 8 ? 3 : QG == 16 ? 4 : 5;
    constexpr int VGL = VG == 8 ? 3 : 4;
    static_assert((1 << QGL) == QG && (1 << VGL) == VG, "power-of-two tiles");
    const int dk_g = dk >> 3, bv_g = bv_here >> 3;
    auto copy_q = [&](int c) { copy_tile(Qs, qg, dk, QGL, dk_g, L, t_begin + c * L); };
    auto copy_kv = [&](int c, int buf) {
        copy_tile(Ks[buf], kg, dk, QGL, dk_g, L, t_begin + c * L);
        copy_tile(Vs[buf], vg + col0, dv, VGL, bv_g, L, t_begin + c * L);
    };

    // ---- gates (wavefront 0; one token per lane)
    float gf = 0.0f, gi = -INFINITY;
    auto load_gates = [&](int c) {
        const int t = t_begin + c * L + lane;
        const bool ok = lane < L && t < t_end;
        const int tc = min(t, t_end - 1);
        const float f = fgg[tc], i = igg[tc];
        gf = ok ? f : 0.0f;
        gi = ok ? i : -INFINITY;
    };
    auto gate_prep = [&](float m_before, float *G) {
        float b = gf;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(b, off, 64);
            if (lane >= off) b += y;
        }
        const float u = gi - b;
        float pm = u;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(pm, off, 64);
            if (lane >= off) pm = fmaxf(pm, y);
        }
        const float r = fmaxf(m_before, pm);
        const float r_last = __shfl(r, L - 1, 64);
        const float b_last = __shfl(b, L - 1, 64);
        if (lane < L) {
            G[lane] = u;
            G[LP + lane] = r;
            G[2 * LP + lane] = exp_e(m_before - r);
            G[3 * LP + lane] = exp_e(-(b + r));
            G[4 * LP + lane] = exp_e(u - r_last);
        }
        if (lane == 0) {
            G[5 * LP + 0] = b_last + r_last;          // stabilizer after the chunk
            G[5 * LP + 1] = exp_e(m_before - r_last); // decay of the carried state
            G[5 * LP + 2] = b_last;                   // sum of log forget gates
        }
    };

    // causal tiles of S owned by this wavefront
    int tjt[MYT], tit[MYT];
    bool tok[MYT];
#pragma unroll
    for (int x = 0; x < MYT; ++x) {
        const int t = wave + NW * x;
        tok[x] = t < NCT;
        int it = 0;
        while ((it + 1) * (it + 2) / 2 <= t) ++it;
        tit[x] = it;
        tjt[x] = t - it * (it + 1) / 2;
    }

    float g_total = 0.0f;
    if (nchunks > 0) {
        __syncthreads();  // zeroing done before the copies land
        if (!STATE_ONLY) copy_q(0);
        copy_kv(0, 0);
        if (wave == 0) {
            load_gates(0);
            gate_prep(m_prev, gt[0]);
        }
        __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        const float *G = gt[buf];
        const int tc = t_begin + c * L;
        const float m_next = G[5 * LP + 0], s_last = G[5 * LP + 1];
        g_total += G[5 * LP + 2];
        const bool more = c + 1 < nchunks;
        const bf16 *K = Ks[buf];
        const bf16 *V = Vs[buf];

        // output-gate inputs of this chunk (rows clamped into the segment)
        uint2 orw[NT][NBT];
        if (!STATE_ONLY) {
#pragma unroll
            for (int it = 0; it < NT; ++it)
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) {
                    const int t = min(tc + 16 * it + l16, t_end - 1);
                    const int b = min(col0 + wcol0 + 16 * bt + 4 * g4, dv - 4);
                    orw[it][bt] = *reinterpret_cast<const uint2 *>(og + (size_t)t * dv + b);
                }
        }
        if (more) {
            if (wave == 0) load_gates(c + 1);
            copy_kv(c + 1, buf ^ 1);
        }

        f32x4 Ot[NBT][NT];
        f32x4 St[MYT];
        f32x4 Qn = {0.f, 0.f, 0.f, 0.f};
        if (!STATE_ONLY) {
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
                for (int it = 0; it < NT; ++it) Ot[bt][it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int x = 0; x < MYT; ++x) St[x] = f32x4{0.f, 0.f, 0.f, 0.f};

            // ---- loop over d_qk: O^T = C'^T Q^T, S^T = K Q^T, qn = Q n'
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                // keep one k-step's fragments live at a time
                __builtin_amdgcn_sched_barrier(0);
                bf16x8 ach[NBT], acl[NBT];
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) {
                    const float x[8] = {Cr[2 * ks][bt][0], Cr[2 * ks][bt][1], Cr[2 * ks][bt][2],
                                        Cr[2 * ks][bt][3], Cr[2 * ks + 1][bt][0], Cr[2 * ks + 1][bt][1],
                                        Cr[2 * ks + 1][bt][2], Cr[2 * ks + 1][bt][3]};
                    split8(x, ach[bt], acl[bt]);
                }
                // n' as a 16-row operand with only row 0 non-zero (this wavefront's token tile)
                bf16x8 anh, anl;
                {
                    const f32x4 n0 = *reinterpret_cast<const f32x4 *>(&nsh[32 * ks + 4 * g4]);
                    const f32x4 n1 = *reinterpret_cast<const f32x4 *>(&nsh[32 * ks + 16 + 4 * g4]);
                    const float z = l16 == 0 ? 1.0f : 0.0f;
                    const float x[8] = {n0[0] * z, n0[1] * z, n0[2] * z, n0[3] * z,
                                        n1[0] * z, n1[1] * z, n1[2] * z, n1[3] * z};
                    split8(x, anh, anl);
                }
#pragma unroll
                for (int it = 0; it < NT; ++it) {
                    const int i = 16 * it + l16;
                    const bf16x8 bq = cat8(
                        *reinterpret_cast<const bf16x4 *>(&Qs[sw_off<QG>(i, 32 * ks + 4 * g4)]),
                        *reinterpret_cast<const bf16x4 *>(&Qs[sw_off<QG>(i, 32 * ks + 16 + 4 * g4)]));
#pragma unroll
                    for (int bt = 0; bt < NBT; ++bt) {
                        Ot[bt][it] = mfma(ach[bt], bq, Ot[bt][it]);
                        Ot[bt][it] = mfma(acl[bt], bq, Ot[bt][it]);
                    }
                    if (it == (wave % NT)) {
                        Qn = mfma(anh, bq, Qn);
                        Qn = mfma(anl, bq, Qn);
                    }
#pragma unroll
                    for (int x = 0; x < MYT; ++x) {
                        if (tok[x] && tit[x] == it) {
                            const int j = 16 * tjt[x] + l16;
                            const bf16x8 ak = cat8(
                                *reinterpret_cast<const bf16x4 *>(&K[sw_off<QG>(j, 32 * ks + 4 * g4)]),
                                *reinterpret_cast<const bf16x4 *>(&K[sw_off<QG>(j, 32 * ks + 16 + 4 * g4)]));
                            St[x] = mfma(ak, bq, St[x]);
                        }
                    }
                }
            }
            // gates of the next chunk (wavefront 0), into the other table
            if (more && wave == 0) gate_prep(m_next, gt[buf ^ 1]);

            // P = S (x) e^{u_j - r_i} -> LDS; column sums -> den_part
#pragma unroll
            for (int x = 0; x < MYT; ++x) {
                if (tok[x]) {
                    const int i = 16 * tit[x] + l16;
                    const float ri = G[LP + i];
                    float p[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * tjt[x] + 4 * g4 + r;
                        p[r] = (j <= i) ? St[x][r] * exp_e(G[j] - ri) : 0.0f;
                    }
                    const bf16x4 pb = {(bf16)p[0], (bf16)p[1], (bf16)p[2], (bf16)p[3]};
                    *reinterpret_cast<bf16x4 *>(&Ps[sw_off<PG>(i, 16 * tjt[x] + 4 * g4)]) = pb;
                    float cs = (p[0] + p[1]) + (p[2] + p[3]);
                    cs += __shfl_xor(cs, 16, 64);
                    cs += __shfl_xor(cs, 32, 64);
                    if (g4 == 0) den_part[(wave + NW * x) * 16 + l16] = cs;
                }
            }
            // q.n' for this wavefront's token tile: row 0 of Qn (lanes g4 == 0, r == 0)
            if (wave < NT && g4 == 0) qn[16 * wave + l16] = Qn[0];
#pragma unroll
            for (int it = 0; it < NT; ++it) {
                const float si = G[2 * LP + 16 * it + l16];
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) Ot[bt][it] *= si;
            }
        } else {
            if (more && wave == 0) gate_prep(m_next, gt[buf ^ 1]);
        }
        __syncthreads();  // (C) P, den_part, qn visible; every wavefront is done with Q
        if (more && !STATE_ONLY) copy_q(c + 1);

        // V^T fragments (token index along k) by transpose reads of the row-major V tile
        // lane (l16, g4): rows j = 32 js + 8 g4 + e (+4), columns b0 + 4 (l16 & 3)
        const int te = l16 >> 2, tq = l16 & 3;
        if (!STATE_ONLY) {
            // ---- O^T += V^T P^T, then h
#pragma unroll
            for (int js = 0; js < NJS; ++js) {
                bf16x8 av[NBT];
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) {
                    const int b0 = wcol0 + 16 * bt + 4 * tq;
                    const int j0 = 32 * js + 8 * g4 + te;
                    av[bt] = cat8(tr_read(&V[sw_off<VG>(j0, b0)]), tr_read(&V[sw_off<VG>(j0 + 4, b0)]));
                }
#pragma unroll
                for (int it = 0; it < NT; ++it) {
                    if (32 * js <= 16 * it + 15) {
                        const int i = 16 * it + l16;
                        const bf16x8 bp = *reinterpret_cast<const bf16x8 *>(&Ps[sw_off<PG>(i, 32 * js + 8 * g4)]);
#pragma unroll
                        for (int bt = 0; bt < NBT; ++bt) Ot[bt][it] = mfma(av[bt], bp, Ot[bt][it]);
                    }
                }
            }
#pragma unroll
            for (int it = 0; it < NT; ++it) {
                const int i = 16 * it + l16;
                const int t = tc + i;
                float den = G[2 * LP + i] * qn[i];
#pragma unroll
                for (int jt = 0; jt <= it; ++jt) den += den_part[(it * (it + 1) / 2 + jt) * 16 + l16];
                const float inv = __builtin_amdgcn_rcpf(fmaxf(fabsf(den), G[3 * LP + i]));
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) {
                    const int b = col0 + wcol0 + 16 * bt + 4 * g4;
                    if (t < t_end && b < dv) {
                        const uint2 o4 = orw[it][bt];
                        float y[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t wd = e < 2 ? o4.x : o4.y;
                            const float ox = __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16));
                            y[e] = Ot[bt][it][e] * inv * __builtin_amdgcn_rcpf(1.0f + exp_e(-ox));
                        }
                        const bf16x4 hv = {(bf16)y[0], (bf16)y[1], (bf16)y[2], (bf16)y[3]};
                        *reinterpret_cast<bf16x4 *>(hg + (size_t)t * dv + b) = hv;
                    }
                }
            }
        }

        // ---- C' <- e^{m - r_last} C' + K^T (w (x) V);  n' <- e^{m - r_last} n' + K^T w
#pragma unroll
        for (int at = 0; at < NAT; ++at)
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) Cr[at][bt] *= s_last;
#pragma unroll
        for (int x = 0; x < NA_W; ++x) Nr[x] *= s_last;
#pragma unroll
        for (int js = 0; js < NJS; ++js) {
            float w8[8];
            {
                const f32x4 w0 = *reinterpret_cast<const f32x4 *>(&G[4 * LP + 32 * js + 8 * g4]);
                const f32x4 w1 = *reinterpret_cast<const f32x4 *>(&G[4 * LP + 32 * js + 8 * g4 + 4]);
                w8[0] = w0[0]; w8[1] = w0[1]; w8[2] = w0[2]; w8[3] = w0[3];
                w8[4] = w1[0]; w8[5] = w1[1]; w8[6] = w1[2]; w8[7] = w1[3];
            }
            bf16x8 bw[NBT];
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) {
                const int b0 = wcol0 + 16 * bt + 4 * tq;
                const int j0 = 32 * js + 8 * g4 + te;
                const bf16x8 vv = cat8(tr_read(&V[sw_off<VG>(j0, b0)]), tr_read(&V[sw_off<VG>(j0 + 4, b0)]));
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = (float)vv[e] * w8[e];
#pragma unroll
                for (int e = 0; e < 8; ++e) bw[bt][e] = (bf16)x[e];
            }
            // w as a 16-column operand with only column 0 non-zero (for n')
            bf16x8 bnh, bnl;
            {
                const float z = l16 == 0 ? 1.0f : 0.0f;
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = w8[e] * z;
                split8(x, bnh, bnl);
            }
#pragma unroll
            for (int at = 0; at < NAT; ++at) {
                if ((at & 3) == 0) __builtin_amdgcn_sched_barrier(0);
                const int a0 = 16 * at + 4 * tq;
                const int j0 = 32 * js + 8 * g4 + te;
                const bf16x8 ak = cat8(tr_read(&K[sw_off<QG>(j0, a0)]), tr_read(&K[sw_off<QG>(j0 + 4, a0)]));
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) Cr[at][bt] = mfma(ak, bw[bt], Cr[at][bt]);
                if (at / NA_W == wave) {
                    Nr[at % NA_W] = mfma(ak, bnh, Nr[at % NA_W]);
                    Nr[at % NA_W] = mfma(ak, bnl, Nr[at % NA_W]);
                }
            }
        }
        // publish n' (column 0 of the n' tiles) for the next chunk's q.n'
        if (l16 == 0) {
#pragma unroll
            for (int x = 0; x < NA_W; ++x)
                *reinterpret_cast<f32x4 *>(&nsh[16 * (wave * NA_W + x) + 4 * g4]) = Nr[x];
        }
        m_prev = m_next;
        __builtin_amdgcn_s_waitcnt(0);  // this chunk's copies of the next chunk have landed
        __syncthreads();                // (D)
    }

    // ---- state out
    float *Cdst = nullptr, *ndst = nullptr, *mdst = nullptr;
    if (STATE_ONLY) {
        float *r = a.seg_out + ((size_t)bh * (a.nseg - 1) + seg) * rec;
        Cdst = r;
        ndst = r + (size_t)dk * dv;
        mdst = ndst + dk;
        if (tile == 0 && tid == 0) mdst[1] = g_total;
    } else if (a.CT && seg == a.nseg - 1) {
        Cdst = a.CT + (size_t)bh * dk * dv;
        ndst = a.nT + (size_t)bh * dk;
        mdst = a.mT + bh;
    }
    if (Cdst) {
#pragma unroll
        for (int at = 0; at < NAT; ++at)
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) {
                const int b = col0 + wcol0 + 16 * bt + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * at + 4 * g4 + r;
                    if (row < dk && b < dv) Cdst[(size_t)row * dv + b] = Cr[at][bt][r];
                }
            }
        if (tile == 0) {
            for (int e = tid; e < dk; e += NTH) ndst[e] = nsh[e];
            if (tid == 0) mdst[0] = m_prev;
        }
    }
}

}  // namespace mlstm
