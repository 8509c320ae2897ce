// prefill_ws.hpp -- chunkwise mLSTM forward for bf16 I/O on gfx950 with the
// wavefronts of a workgroup split by role.
//
// Mathematics as in prefill_kernel.hpp (the chunkwise form of the xLSTM
// note's mLSTM recurrence, "mLSTM (matrix LSTM)" section, with the
// stabilizer of its "sLSTM" section): per chunk of L = 64 tokens, with
// b = in-chunk cumsum of f~, u_j = i~_j - b_j, r_i = max(m, max_{j<=i} u_j),
//   h_i = sigmoid(o~_i) (sum_j P_ij v_j + e^{m-r_i} C'^T q_i)
//                       / max(|sum_j P_ij + e^{m-r_i} n'.q_i|, e^{-(b_i+r_i)}),
//   P_ij = (q_i.k_j) e^{u_j - r_i} (j <= i),
//   C' <- e^{m-r_L} C' + sum_j e^{u_j-r_L} k_j v_j^T, n' likewise, m <- b_L + r_L.
//
// Schedule.  One workgroup owns one (pair, segment, block of 128 value
// columns) and walks its chunks in order.  Its 8 wavefronts sit two per SIMD,
// one of each role, so the matrix cores of a SIMD run one role's MFMAs while
// its vector ALU runs the other role's elementwise work:
//  * state wavefronts (0..3): wavefront s holds all d_qk rows of C' for value
//    columns [32 s, 32 s + 32) in registers (MFMA accumulator layout, float32,
//    for the whole sequence).  Per chunk they compute the inter-chunk
//    read-out C'^T Q^T (C' split into a bf16 high part and remainder, two
//    MFMAs) and hand it to the intra wavefronts through LDS, then update C'
//    and n' with one straight run of MFMAs.  They issue no memory
//    instructions (a wavefront whose vector-memory queue is full stalls at
//    issue);
//  * intra wavefronts (4..7): wavefront 4 + t owns token tile t (16 tokens)
//    for all 128 columns: its causal S tiles (MFMA), P in registers (the S
//    accumulator layout is, up to a permutation of the MFMA k index that the
//    V^T fragment follows too, the B operand of V^T P^T), V^T P^T, q.n' (MFMA
//    with n' as a broadcast operand), the normaliser, the output gate and
//    the bf16 h stores.  They copy the Q, K and V tiles.
// Two phases per chunk, separated by workgroup barriers:
//   phase 1: state: read-out of chunk c -> LDS
//            intra: copy V(c), load o~, gates; S, q.n', P of chunk c; one of
//                   them prepares the gate table of chunk c+1; copy K(c+1)
//   phase 2: state: C', n' update with chunk c (n' double buffered: the
//                   intra wavefronts read the other one in phase 1)
//            intra: copy Q(c+1); V^T P^T on top of the read-out, h of chunk c
// No wavefront has a copy in flight when it uses a plain load (the compiler
// counts loads and copies together and would wait for both); the barriers
// wait for the copies with exact counts.
#pragma once

#include "prefill_bf16.hpp"

namespace mlstm {

template <int DKP_>
struct WsCfg {
    static constexpr int L = 64, DKP = DKP_, BV = 128;
    static constexpr int NW = 8, NTH = 512, NSW = 4;  // wavefronts; state wavefronts
    static constexpr int NT = L / 16;                 // token tiles (one per intra wavefront)
    static constexpr int NAT = DKP / 16;              // 16-row tiles of C'
    static constexpr int NKS = DKP / 32;              // MFMA k-steps over d_qk
    static constexpr int NCT = BV / 16;               // 16-column tiles of the value block
    static constexpr int QG = DKP / 8, VG = BV / 8;   // 16-byte granules per row
    static constexpr int GTF = 6 * L + 8;             // gate table floats (as Bf16Cfg)
    static constexpr size_t LDS_BYTES = 2 * (3 * (size_t)L * DKP + (size_t)L * BV) +
                                        16 * (size_t)NT * NCT * 64 + 4 * (2 * (size_t)GTF + 2 * (size_t)DKP) +
                                        2 * 2 * 2 * (size_t)DKP + 2 * (size_t)L;
    static_assert(NT == NW - NSW, "one token tile per intra wavefront");
    static_assert(NAT % 4 == 0, "n' tiles spread over the state wavefronts");
    static_assert(QG >= 8, "swizzle needs 8 granules per row");
};

// Row swizzles of the 16-byte granules of the Q, K and V tiles.  Two kinds
// of read must spread over the LDS banks:
//  * fragment reads (Q, K): 16 consecutive rows, one whole granule each, at
//    the same logical granule;
//  * transpose reads (K, V): four rows 4 g + (0..3) or 8 g + (0..3), 8-byte
//    halves of four consecutive logical granules 4 a + (0..3), all at the
//    same half.
// With 16 or more granules per row (rows a multiple of 256 bytes apart, so a
// granule's banks depend on its position only) swzt16 swaps the two 2-bit
// digits of row mod 16: a bijection of row mod 16 (fragment reads), and rows
// 0..3 of an 8-row group differ in bits 2-3 (the four granules of a transpose
// read then land in four different aligned groups of four).  With 8 granules
// per row (128-byte rows: odd rows sit half the banks over) swzt8 reverses
// the bits of (row / 2) mod 8: a bijection over the 8 rows of each parity,
// and rows two apart differ in bit 2.
__device__ __forceinline__ int swzt16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swzt8(int r) {
    const int x = (r >> 1) & 7;
    return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
}

typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// word 3 of the buffer descriptors of the tile copies, output-gate loads and
// h stores (32-bit data format; raw addressing, range-checked)
constexpr int kWsBuf = 0x00020000;

// Split 8 floats into bf16 high parts and bf16 remainders, both rounded to
// nearest even and converted in pairs.  The remainder x - hi is exact in
// float32: the high parts are unpacked by a shift and a mask and subtracted.
// Six instructions per pair, two of them conversions (on gfx950 conversion and
// dot-product instructions make no progress while the matrix core runs the
// other wavefront's MFMAs on this SIMD; plain ALU instructions do).
__device__ __forceinline__ void split8_rr(const float *x, bf16x8 &hi, bf16x8 &lo) {
    bf16x2 h[4], l[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const f32x2 v = {x[2 * p], x[2 * p + 1]};
        h[p] = __builtin_convertvector(v, bf16x2);
        const unsigned hb = __builtin_bit_cast(unsigned, h[p]);
        const f32x2 r = {v.x - __uint_as_float(hb << 16), v.y - __uint_as_float(hb & 0xffff0000u)};
        l[p] = __builtin_convertvector(r, bf16x2);
    }
    hi = bf16x8{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
    lo = bf16x8{l[0][0], l[0][1], l[1][0], l[1][1], l[2][0], l[2][1], l[3][0], l[3][1]};
}

// One of four fragments, chosen by a wavefront-uniform index given as bit
// masks m0, m1 (each 0 or all ones): two levels of bitwise selects, twelve
// VALU instructions.  Masks rather than booleans, because a select on a
// uniform boolean is turned into a branch, which splits the MFMA run.
__device__ __forceinline__ bf16x8 pick4(const bf16x8 &f0, const bf16x8 &f1, const bf16x8 &f2, const bf16x8 &f3,
                                        unsigned m0, unsigned m1) {
    const u32x4 a0 = __builtin_bit_cast(u32x4, f0), a1 = __builtin_bit_cast(u32x4, f1);
    const u32x4 a2 = __builtin_bit_cast(u32x4, f2), a3 = __builtin_bit_cast(u32x4, f3);
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned lo = (m0 & a1[i]) | (~m0 & a0[i]);
        const unsigned hi = (m0 & a3[i]) | (~m0 & a2[i]);
        r[i] = (m1 & hi) | (~m1 & lo);
    }
    return __builtin_bit_cast(bf16x8, r);
}

// Swizzle of a tile with GPR granules per row (Q, K and V tiles alike).
template <int GPR>
__device__ __forceinline__ int tswz(int r) {
    if constexpr (GPR >= 16)
        return swzt16(r);
    else
        return swzt8(r);
}

// Workgroup barrier after this wavefront's LDS accesses have completed and at
// most VM of its vector-memory operations are outstanding (they complete in
// issue order).  State wavefronts issue none and pass VM = 63 (no wait).
template <int VM>
__device__ __forceinline__ void role_sync() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 0xf) | (0x7 << 4) | (0x0 << 8) | ((VM >> 4) << 14));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// SO (state only): the segment scan's first pass -- each segment's local
// state from the zero state, no output.  The state wavefronts run the C'
// update alone; the intra wavefronts copy K and V (both double buffered, the
// second V buffer in the unused exchange area), prepare the gates and update
// n', one barrier per chunk.
template <int DKP, bool SO>
__global__ __launch_bounds__(512, 1) void mlstm_ws_kernel(FwdArgs a) {
    using Cfg = WsCfg<DKP>;
    constexpr int L = Cfg::L, LP = L, BV = Cfg::BV, NSW = Cfg::NSW, NT = Cfg::NT;
    constexpr int NAT = Cfg::NAT, NKS = Cfg::NKS, NCT = Cfg::NCT, QG = Cfg::QG, VG = Cfg::VG;
    constexpr int GTF = Cfg::GTF;
    constexpr int NHS = NCT / 2;  // 16-byte h stores (and output-gate loads) per lane per chunk
    constexpr float kRenorm = 8.6736174e-19f;  // 2^-60: renormalise the lazy state scale below this

    __shared__ __attribute__((aligned(16))) bf16 Qs[L * DKP];
    __shared__ __attribute__((aligned(16))) bf16 Ks[2][L * DKP];  // K of even / odd chunks
    __shared__ __attribute__((aligned(16))) bf16 Vs[L * BV];
    __shared__ __attribute__((aligned(16))) f32x4 Xch[NT][NCT][64];  // scaled read-out, accumulator layout
    // gate tables (double buffered): u, r (times log2 e), s, floor, w [L] floats, w as bf16
    // high/low pairs [L], then scalars (m after, decay, sum f~)
    __shared__ __attribute__((aligned(16))) float gt[2][GTF];
    // n' (true scale) and as bf16 high part and remainder, double buffered
    // (buffer c & 1 holds n' before chunk c)
    __shared__ __attribute__((aligned(16))) float nsh[2][DKP];
    __shared__ __attribute__((aligned(16))) bf16 nhl[2][2][DKP];
    // zeros: the B operand columns of the n' update other than its group's
    __shared__ __attribute__((aligned(16))) bf16 nzero[L];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_state = wave < NSW;
    const int s = wave & 3;  // state: column group; intra: token tile
    const int l16 = lane & 15, g4 = lane >> 4;
    const int te = l16 >> 2, tq = l16 & 3;  // transpose-read source row / column quad

    const int nwg = gridDim.x;
    int logical = blockIdx.x;
    if ((nwg & 7) == 0) logical = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int gseg = SO ? a.nseg - 1 : a.nseg;  // segments this launch covers
    const int tile = logical % a.ntile;
    const int rest = logical / a.ntile;
    const int seg = rest % gseg;
    const int bh = rest / gseg;

    const int dk = a.dk, dv = a.dv, T = a.T;  // here dk == DKP and dv is a multiple of BV
    const int t_begin = seg * a.seg_len;
    const int t_end = min(t_begin + a.seg_len, T);
    const int nchunks = (t_end - t_begin + L - 1) / L;
    const int col0 = tile * BV;

    // input rows in the call's layout (ldq, ldv elements apart), h dense
    const int ldq = a.lq.ld, ldv = a.lv.ld;
    const bf16 *qg = static_cast<const bf16 *>(a.q) + row_base(a.lq, bh);
    const bf16 *kg = static_cast<const bf16 *>(a.k) + row_base(a.lq, bh);
    const bf16 *vg = static_cast<const bf16 *>(a.v) + row_base(a.lv, bh) + col0;
    const bf16 *og = static_cast<const bf16 *>(a.o) + row_base(a.lv, bh) + col0;
    bf16 *hg = static_cast<bf16 *>(a.h) + (size_t)bh * T * dv + col0;
    const float *igg = a.ig + (size_t)bh * T;
    const float *fgg = a.fg + (size_t)bh * T;

    for (int e = tid; e < 2 * GTF; e += Cfg::NTH) (&gt[0][0])[e] = 0.0f;
    for (int e = tid; e < L; e += Cfg::NTH) nzero[e] = (bf16)0.0f;

    // ---- initial state
    const size_t rec = seg_state_floats(dk, dv);
    const float *Cs = nullptr, *ns = nullptr;
    float m_prev = 0.0f;
    if (SO) {
        m_prev = -1e30f;  // no past: the first chunk's stabilizer comes from its own gates
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
    // Value columns.  Row i = 4 g + r of a 16-column tile cb (V^T fragments,
    // read-out and output accumulators) and column i of C' tile bt = cb - 2 s
    // stand for value column 32 (cb / 2) + 8 g + 4 (cb % 2) + r: tiles 2 m
    // and 2 m + 1 together give each lane group 8 consecutive columns, so h
    // and the output gate move 16 bytes per lane.
    const int scol = col0 + 32 * s + 8 * te + tq;  // state column of this lane (tile bt adds 4 bt)
    // Row i = 4 g4 + r of the 16-row C' tile at holds d_qk index
    // 32 (at / 2) + 8 g4 + 4 (at % 2) + r: tiles 2 kk and 2 kk + 1 together give
    // each lane group 8 consecutive d_qk indices, the k slots of one whole Q
    // granule in the read-out.  The K^T fragments of the update follow it.
    auto crow = [&](int at, int r) -> int { return 32 * (at >> 1) + 8 * g4 + 4 * (at & 1) + r; };
    f32x4 Cr[NAT][2];
#pragma unroll
    for (int at = 0; at < NAT; ++at)
#pragma unroll
        for (int bt = 0; bt < 2; ++bt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Cr[at][bt][r] = (is_state && Cs) ? Cs[(size_t)crow(at, r) * dv + scol + 4 * bt] : 0.0f;
    for (int e = tid; e < DKP; e += Cfg::NTH) {
        const float x = ns ? ns[e] : 0.0f;
        nsh[0][e] = x;
        const bf16 hi = (bf16)x;
        nhl[0][0][e] = hi;
        nhl[0][1][e] = (bf16)(x - (float)hi);
    }
    float sigma = 1.0f;  // C' is held divided by sigma (state wavefronts)

    auto qswz = [](int row) -> int { return tswz<QG>(row); };
    // ---- global -> LDS copies by the intra wavefronts.  Physical granule g
    // of a tile is (row, p) with p = g % gpr holding logical granule
    // p ^ swz(row); instruction k of wavefront s fills granules
    // [(k NSW + s) 64, +64), rows k RPI + const.  The per-lane part of
    // instruction k's source offset is off[k % 2] (bytes; the swizzle repeats
    // every 16 rows and 2 RPI is a multiple of 16) from a base (k - k % 2) RPI
    // rows further, so each pair of instructions reads through one buffer
    // descriptor (scalar registers: no per-lane 64-bit address arithmetic)
    // whose range ends at the segment's last row.  Rows past it read as zero
    // (finite; their gates zero them out).  The whole offset is the per-lane
    // one: the range check covers it.  gpr_c: granules per row of the tile
    // (its swizzle follows from it).
    auto copy_offsets = [&](auto gpr_c, int ld, unsigned *off) {
        constexpr unsigned GPR = decltype(gpr_c)::value;
        constexpr unsigned RPI = NSW * 64 / GPR;
        static_assert((L * GPR) % (NSW * 64) == 0 && (2 * RPI) % 16 == 0, "copy shape, swizzle period");
        const unsigned pgr = (unsigned)s * 64u + (unsigned)lane;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const unsigned row = k * RPI + pgr / GPR;
            off[k] = 2u * (row * (unsigned)ld + ((pgr % GPR) ^ (unsigned)tswz<GPR>((int)row)) * 8u);
        }
    };
    auto copy_tile = [&](bf16 *dst, const bf16 *src, int ld, auto gpr_c, int tc, const unsigned *off) {
        constexpr int GPR = decltype(gpr_c)::value;
        constexpr int NI = L * GPR / (NSW * 64), RPI = NSW * 64 / GPR;
        static_assert(NI % 2 == 0, "instructions in pairs");
#pragma unroll
        for (int k = 0; k < NI; k += 2) {
            const int r0 = tc + k * RPI;
            // (uniform; readfirstlane keeps the clamp's result in a scalar
            // register, which the descriptor needs)
            const int nb = __builtin_amdgcn_readfirstlane(max(0, min(2 * RPI, t_end - r0)) * ld * 2);
            const auto rs = __builtin_amdgcn_make_buffer_rsrc((void *)(src + (size_t)r0 * ld), 0, nb, kWsBuf);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + ((k + j) * NSW + s) * 64 * 8), 16,
                                                         off[j], 0, 0, 0);
        }
    };
    static_assert(L * QG / (NSW * 64) == NKS, "one K or Q copy instruction per d_qk k-step");
    using QGc = std::integral_constant<int, QG>;
    using VGc = std::integral_constant<int, VG>;

    // V tile of chunk c (state-only: double buffered, odd chunks in Xch)
    auto vbuf = [&](int c) -> bf16 * { return (SO && (c & 1)) ? reinterpret_cast<bf16 *>(&Xch[0][0][0]) : Vs; };
    static_assert(sizeof(Xch) >= sizeof(Vs), "second V buffer");

    // ---- gates (first intra wavefront; one token per lane)
    constexpr int GW = NSW;
    float gf = 0.0f, gi = -INFINITY;
    bool gok = false;
    auto load_gates = [&](int c) {
        const int t = t_begin + c * L + lane;
        gok = lane < L && t < t_end;
        const int tcl = min(t, t_end - 1);
        gf = fgg[tcl];
        gi = igg[tcl];
    };
    auto gate_prep = [&](float m_before, float *G) {
        const float b = wave_scan_add(gok ? gf : 0.0f);
        const float u = (gok ? gi : -INFINITY) - b;
        const float pm = wave_scan_max(u);
        const float r = fmaxf(m_before, pm);
        const float r_last = __shfl(r, L - 1, 64);
        const float b_last = __shfl(b, L - 1, 64);
        const float w = exp_e(u - r_last);
        // u and r in base-2 units: P's weights are then one exp2 of a difference
        G[lane] = u * 1.4426950408889634f;
        G[LP + lane] = r * 1.4426950408889634f;
        G[2 * LP + lane] = exp_e(m_before - r);
        G[3 * LP + lane] = exp_e(-(b + r));
        G[4 * LP + lane] = w;
        const bf16 whi = (bf16)w;
        const bf16 wlo = (bf16)(w - (float)whi);
        bf16 *W2 = reinterpret_cast<bf16 *>(&G[5 * LP]);
        W2[lane] = whi;
        W2[LP + lane] = wlo;
        if (lane == 0) {
            G[6 * LP + 0] = b_last + r_last;           // stabilizer after the chunk
            G[6 * LP + 1] = exp_e(m_before - r_last);  // decay of the carried state
            G[6 * LP + 2] = b_last;                    // sum of the chunk's log forget gates
        }
    };

    // ---- per-lane LDS offsets
    // Q / K fragment for k-step ks of rows 16 t + l16: columns 32 ks + 8 g4
    // .. +8, i.e. the whole logical granule 4 ks + g4; the swizzle touches the
    // low four granule bits, so the per-lane part depends on ks & 3 and
    // ks >> 2 adds 16 granules (128 elements)
    constexpr int NQO = NKS < 4 ? NKS : 4;
    const int s16 = qswz(l16);
    int qkoff[NQO];
#pragma unroll
    for (int par = 0; par < NQO; ++par) qkoff[par] = l16 * DKP + (((4 * par + g4) ^ s16) << 3);
    auto qk_frag = [&](const bf16 *tilebase, int ks) -> bf16x8 {  // tilebase: row 16 t of the tile
        return *reinterpret_cast<const bf16x8 *>(tilebase + ((ks >> 2) << 7) + qkoff[ks & 3]);
    };
    // Transpose read of value-column tile cb of a V tile row: the lanes of
    // column quad tq supply fragment rows 4 tq .. 4 tq + 3, value columns
    // 32 (cb / 2) + 8 tq + 4 (cb % 2) + (0..3): half cb % 2 of logical granule
    // 4 (cb / 2) + tq.  vtr_off gives the offset without the half.
    auto vtr_off = [](int row, int m, int q) -> int {
        return row * VG * 8 + (((4 * m + q) ^ tswz<VG>(row)) << 3);
    };
    // k index in the S accumulator order (V^T of V^T P^T): rows 32 js + 4 g4 + te (+16)
    const int prow0 = 4 * g4 + te, prow1 = prow0 + 16;

    // n' <- decay n' + K^T w (true scale) from buffer nb into nb ^ 1, for the
    // row tiles s + 4 x, by wavefront s of the intra role: the state-only
    // pass's update of n', run beside the state wavefronts' C' update (which
    // reads the same K tile).  MFMAs with w's high part and remainder in every
    // column of the B operand, on K^T fragments read per k-step.
    auto nprime_intra = [&](const bf16 *K, const float *G, float s_last, int nb) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int lte = (ln & 15) >> 2, ltq = ln & 3, lg4 = ln >> 4;
        const int krow0 = 8 * lg4 + lte, krow1 = krow0 + 4;
        const int kb0 = krow0 * QG * 8, kb1 = krow1 * QG * 8;
        const int kx0 = qswz(krow0) ^ ltq, kx1 = qswz(krow1) ^ ltq;
        const bf16 *W2 = reinterpret_cast<const bf16 *>(&G[5 * LP]);
        constexpr int NX = NAT / 4;
        f32x4 nh[NX], nl[NX];
#pragma unroll
        for (int x = 0; x < NX; ++x) nh[x] = nl[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int js = 0; js < L / 32; ++js) {
            const bf16 *k0 = K + 32 * js * DKP;
            bf16x8 af[NX];
#pragma unroll
            for (int x = 0; x < NX; ++x) {
                const int at = 4 * x + s;
                const int h = 4 * (at & 1), g = 4 * (at >> 1);
                af[x] = cat8(tr_read(k0 + kb0 + h + ((g ^ kx0) << 3)), tr_read(k0 + kb1 + h + ((g ^ kx1) << 3)));
            }
            const bf16x8 bnh = *reinterpret_cast<const bf16x8 *>(W2 + 32 * js + 8 * lg4);
            const bf16x8 bnl = *reinterpret_cast<const bf16x8 *>(W2 + LP + 32 * js + 8 * lg4);
#pragma unroll
            for (int x = 0; x < NX; ++x) nh[x] = mfma(af[x], bnh, nh[x]);
#pragma unroll
            for (int x = 0; x < NX; ++x) nl[x] = mfma(af[x], bnl, nl[x]);
        }
        if (l16 == 0) {
#pragma unroll
            for (int x = 0; x < NX; ++x) {
                const int r0 = crow(s + 4 * x, 0);
                *reinterpret_cast<f32x4 *>(&nsh[nb ^ 1][r0]) =
                    *reinterpret_cast<const f32x4 *>(&nsh[nb][r0]) * s_last + (nh[x] + nl[x]);
            }
        }
    };

    if (nchunks > 0) block_sync<0>();  // gate tables zeroed, n' written

    // Each role runs its own chunk loop; both execute the same sequence of
    // barriers (one after the prologue, two per chunk).
    if (is_state) {
        // ========================= state wavefronts =========================
        // C'/sigma' += K^T ((w/sigma') (x) V) with sigma' = sigma * decay, and
        // n' (true scale) from buffer nb into nb ^ 1: the update with the chunk
        // whose K and V tiles and gate table are given.  The loop over the row
        // tiles of C' is one straight run of MFMAs: n' rides along without a
        // branch (a branch per row tile doubles the update's time).
        auto update = [&](const bf16 *K, const bf16 *Vt, const float *G, float s_last, int nb) {
                sigma *= s_last;
                if (sigma < kRenorm) {  // uniform: fold sigma back into the held state
    #pragma unroll
                    for (int at = 0; at < NAT; ++at)
    #pragma unroll
                        for (int bt = 0; bt < 2; ++bt) Cr[at][bt] *= sigma;
                    sigma = 1.0f;
                }
                const float rsig = __builtin_amdgcn_rcpf(sigma);
                // K^T fragment offsets by (row tile & 3, read), recomputed here from
                // an opaque copy of the lane index so they are not held across the loop
                int ln = lane;
                asm volatile("" : "+v"(ln));
                const int lte = (ln & 15) >> 2, ltq = ln & 3, lg4 = ln >> 4;
                const int krow0 = 8 * lg4 + lte, krow1 = krow0 + 4;
                // K^T row tile at: the lanes of column quad tq supply fragment rows
                // 4 tq .. 4 tq + 3, here d_qk 32 (at / 2) + 8 tq + 4 (at % 2) + (0..3):
                // half at % 2 of logical granule 4 (at / 2) + tq of rows krow0 / krow1
                const int kb0 = krow0 * QG * 8, kb1 = krow1 * QG * 8;
                const int kx0 = qswz(krow0) ^ ltq, kx1 = qswz(krow1) ^ ltq;
                auto kt_frag = [&](const bf16 *rowblock, int at) -> bf16x8 {
                    const int h = 4 * (at & 1), g = 4 * (at >> 1);
                    return cat8(tr_read(rowblock + kb0 + h + ((g ^ kx0) << 3)),
                                tr_read(rowblock + kb1 + h + ((g ^ kx1) << 3)));
                };
                // n' of row tiles s + 4 x (x < NXG): K^T w as MFMAs whose B
                // operand holds w (high part, then remainder) in column x only,
                // zeros elsewhere, all groups into one pair of accumulators, so
                // that lane (x, g4) ends with group x's rows 4 g4 .. 4 g4 + 3
                // and the lanes x < NXG finish one group each; the old value is
                // read now, used at the end.  The row tile is picked from the
                // last four fragments by selects on the wavefront index.
                // (full pass only: in the state-only pass the otherwise idle
                // intra wavefronts update n', with nprime_intra)
                constexpr int NXG = NAT / 4;
                unsigned sm0 = 0u - (unsigned)(s & 1), sm1 = 0u - (unsigned)((s >> 1) & 1);
                asm volatile("" : "+s"(sm0), "+s"(sm1));
                f32x4 nold = {0.f, 0.f, 0.f, 0.f}, nacc_h = {0.f, 0.f, 0.f, 0.f}, nacc_l = nacc_h;
                if constexpr (!SO) nold = *reinterpret_cast<const f32x4 *>(&nsh[nb][crow(s + 4 * (l16 < NXG ? l16 : 0), 0)]);
    #pragma unroll
                for (int js = 0; js < L / 32; ++js) {
                    const bf16 *k0 = K + 32 * js * DKP;
                    float w8[8];
                    {
                        const f32x4 w0 = *reinterpret_cast<const f32x4 *>(&G[4 * LP + 32 * js + 8 * g4]);
                        const f32x4 w1 = *reinterpret_cast<const f32x4 *>(&G[4 * LP + 32 * js + 8 * g4 + 4]);
    #pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            w8[e] = w0[e] * rsig;
                            w8[e + 4] = w1[e] * rsig;
                        }
                    }
                    bf16x8 bw[2];
                    const bf16 *vb = Vt + 32 * js * BV;
                    const int vo0 = vtr_off(krow0, s, ltq), vo1 = vtr_off(krow1, s, ltq);
    #pragma unroll
                    for (int bt = 0; bt < 2; ++bt) {  // value-column tile 2 s + bt
                        const bf16x8 vv = cat8(tr_read(vb + vo0 + 4 * bt), tr_read(vb + vo1 + 4 * bt));
    #pragma unroll
                        for (int e = 0; e < 8; ++e) bw[bt][e] = (bf16)((float)vv[e] * w8[e]);
                    }
                    const bf16 *W2 = reinterpret_cast<const bf16 *>(&G[5 * LP]);
                    bf16x8 bnh[NXG], bnl[NXG];
                    if constexpr (!SO) {
    #pragma unroll
                        for (int x = 0; x < NXG; ++x) {
                            const bool mine = l16 == x;
                            const bf16 *sh = mine ? W2 : nzero, *sl = mine ? W2 + LP : nzero;
                            bnh[x] = *reinterpret_cast<const bf16x8 *>(sh + 32 * js + 8 * g4);
                            bnl[x] = *reinterpret_cast<const bf16x8 *>(sl + 32 * js + 8 * g4);
                        }
                    }
                    // K^T fragments fetched four row tiles ahead (the reads'
                    // latency under load is several MFMA pairs), in a ring of
                    // eight that still holds a group of four when it completes
                    constexpr int AHEAD = 4;
                    bf16x8 ak[8];
    #pragma unroll
                    for (int u = 0; u < AHEAD; ++u) ak[u] = kt_frag(k0, u);
    #pragma unroll
                    for (int at = 0; at < NAT; ++at) {
                        __builtin_amdgcn_sched_barrier(0);
                        if (at + AHEAD < NAT) ak[(at + AHEAD) & 7] = kt_frag(k0, at + AHEAD);
                        const bf16x8 &a0 = ak[at & 7];
    #pragma unroll
                        for (int bt = 0; bt < 2; ++bt) Cr[at][bt] = mfma(a0, bw[bt], Cr[at][bt]);
                        if (!SO && (at & 3) == 3) {  // compile-time: the group at - 3 .. at is complete
                            const bf16x8 fn = pick4(ak[(at - 3) & 7], ak[(at - 2) & 7], ak[(at - 1) & 7], a0, sm0, sm1);
                            nacc_h = mfma(fn, bnh[at >> 2], nacc_h);
                            nacc_l = mfma(fn, bnl[at >> 2], nacc_l);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                // n' <- decay n' + K^T w into buffer nb ^ 1 (read after barrier Y)
                if (!SO && l16 < NXG) {  // lane (x, g4): rows 4 g4 .. +3 of group x = l16
                    const int r0 = crow(s + 4 * l16, 0);
                    const f32x4 nn = nold * s_last + (nacc_h + nacc_l);
                    *reinterpret_cast<f32x4 *>(&nsh[nb ^ 1][r0]) = nn;
                    bf16x4 hi, lo;
    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        hi[r] = (bf16)nn[r];
                        lo[r] = (bf16)(nn[r] - (float)hi[r]);
                    }
                    *reinterpret_cast<bf16x4 *>(&nhl[nb ^ 1][0][r0]) = hi;
                    *reinterpret_cast<bf16x4 *>(&nhl[nb ^ 1][1][r0]) = lo;
                }
        };
        role_sync<63>();
        float g_total = 0.0f;  // sum of the segment's log forget gates (state-only)
        if constexpr (SO) {
            for (int c = 0; c < nchunks; ++c) {
                const float *G = gt[c & 1];
                const float m_next = G[6 * LP + 0], s_last = G[6 * LP + 1];
                g_total += G[6 * LP + 2];
                update(Ks[c & 1], vbuf(c), G, s_last, c & 1);
                m_prev = m_next;
                role_sync<63>();  // K(c+1), V(c+1), gates of c+1 landed; K(c), V(c) free
            }
        }
        for (int c = 0; c < (SO ? 0 : nchunks); ++c) {
            const float *G = gt[c & 1];
            const float m_next = G[6 * LP + 0], s_last = G[6 * LP + 1];

            // ---- phase 1: read-out O^T = C'^T Q^T
            {
                f32x4 Ot[2][NT];
#pragma unroll
                for (int bt = 0; bt < 2; ++bt)
#pragma unroll
                    for (int t = 0; t < NT; ++t) Ot[bt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
                // the Q fragments of a k-step stay in registers for the high
                // and the low pass; the low pass refills each for the next
                // k-step
                bf16x8 qf[NT];
#pragma unroll
                for (int t = 0; t < NT; ++t) qf[t] = qk_frag(Qs + 16 * t * DKP, 0);
#pragma unroll
                for (int kk = 0; kk < NKS; ++kk) {
                    __builtin_amdgcn_sched_barrier(0);
                    bf16x8 ach[2], acl[2];
#pragma unroll
                    for (int bt = 0; bt < 2; ++bt) {
                        const float x[8] = {Cr[2 * kk][bt][0],     Cr[2 * kk][bt][1],     Cr[2 * kk][bt][2],
                                            Cr[2 * kk][bt][3],     Cr[2 * kk + 1][bt][0], Cr[2 * kk + 1][bt][1],
                                            Cr[2 * kk + 1][bt][2], Cr[2 * kk + 1][bt][3]};
                        split8_rr(x, ach[bt], acl[bt]);
                    }
#pragma unroll
                    for (int t = 0; t < NT; ++t)
#pragma unroll
                        for (int bt = 0; bt < 2; ++bt) Ot[bt][t] = mfma(ach[bt], qf[t], Ot[bt][t]);
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
#pragma unroll
                        for (int bt = 0; bt < 2; ++bt) Ot[bt][t] = mfma(acl[bt], qf[t], Ot[bt][t]);
                        if (kk + 1 < NKS) qf[t] = qk_frag(Qs + 16 * t * DKP, kk + 1);
                    }
                }
                // scale by e^{m - r_i} and the held state's sigma, hand over
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const float si = G[2 * LP + 16 * t + l16] * sigma;
#pragma unroll
                    for (int bt = 0; bt < 2; ++bt) Xch[t][2 * s + bt][lane] = Ot[bt][t] * si;
                }
            }
            role_sync<63>();  // (X) read-out in LDS; V(c) landed; Q(c) free

            update(Ks[c & 1], Vs, G, s_last, c & 1);
            m_prev = m_next;
            role_sync<63>();  // (Y) Q(c+1), K(c+1) landed; n' after c written; V(c), Xch free
        }

        // ---- state out (n' and m from wavefront 0 of column block 0): the
        // final state, or (state-only) the segment's local state record
        float *Cdst = nullptr, *ndst = nullptr, *mdst = nullptr;
        if (SO) {
            float *r = a.seg_out + ((size_t)bh * (a.nseg - 1) + seg) * rec;
            Cdst = r;
            ndst = r + (size_t)dk * dv;
            mdst = ndst + dk;
            if (tile == 0 && wave == 0 && lane == 0) mdst[1] = g_total;
        } else if (a.CT && seg == a.nseg - 1) {
            Cdst = a.CT + (size_t)bh * dk * dv;
            ndst = a.nT + (size_t)bh * dk;
            mdst = a.mT + bh;
        }
        if (Cdst) {
#pragma unroll
            for (int at = 0; at < NAT; ++at)
#pragma unroll
                for (int bt = 0; bt < 2; ++bt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Cdst[(size_t)crow(at, r) * dv + scol + 4 * bt] = Cr[at][bt][r] * sigma;
            if (tile == 0 && wave == 0) {
                for (int e = lane; e < dk; e += 64) ndst[e] = nsh[nchunks & 1][e];
                if (lane == 0) mdst[0] = m_prev;
            }
        }
    } else {
        // ========================= intra wavefronts =========================
        unsigned qko[2], vo[2];  // per-lane copy offsets of Q/K and V tiles
        copy_offsets(QGc{}, ldq, qko);
        copy_offsets(VGc{}, ldv, vo);
        if constexpr (SO) {
            if (nchunks > 0) {
                copy_tile(Ks[0], kg, ldq, QGc{}, t_begin, qko);
                copy_tile(vbuf(0), vg, ldv, VGc{}, t_begin, vo);
                if (wave == GW) {
                    load_gates(0);
                    gate_prep(m_prev, gt[0]);
                }
            }
            role_sync<0>();
            for (int c = 0; c < nchunks; ++c) {
                if (c + 1 < nchunks) {
                    const int tn = t_begin + (c + 1) * L;
                    if (wave == GW) load_gates(c + 1);
                    copy_tile(Ks[(c + 1) & 1], kg, ldq, QGc{}, tn, qko);
                    copy_tile(vbuf(c + 1), vg, ldv, VGc{}, tn, vo);
                    if (wave == GW) gate_prep(gt[c & 1][6 * LP + 0], gt[(c + 1) & 1]);
                }
                // n' with chunk c while its copies of chunk c + 1 are in flight
                nprime_intra(Ks[c & 1], gt[c & 1], gt[c & 1][6 * LP + 1], c & 1);
                role_sync<0>();  // K(c+1), V(c+1) landed, gates of c+1 and n' after c written
            }
            return;
        }
        if (nchunks > 0) {
            copy_tile(Qs, qg, ldq, QGc{}, t_begin, qko);
            copy_tile(Ks[0], kg, ldq, QGc{}, t_begin, qko);
            if (wave == GW) {
                load_gates(0);
                gate_prep(m_prev, gt[0]);
            }
        }
        role_sync<0>();
        const int it = s;                // token tile of this wavefront
        const int irow = 16 * it + l16;  // token of this lane within the chunk (accumulator column)
        for (int c = 0; c < nchunks; ++c) {
            const float *G = gt[c & 1];
            float *Gnext = gt[(c + 1) & 1];
            const int tc = t_begin + c * L;
            const float m_next = G[6 * LP + 0];
            const bool more = c + 1 < nchunks;

            // ---- phase 1: copy V(c); S, P of this token tile; next gate
            // table; copy K(c+1)
            copy_tile(Vs, vg, ldv, VGc{}, tc, vo);
            // this chunk's rows of o~ and h: buffer descriptors whose range ends
            // at the segment's last row (o~ past it reads as zero, h past it is
            // not written)
            const int nrow = __builtin_amdgcn_readfirstlane(min(L, t_end - tc));
            const auto ro = __builtin_amdgcn_make_buffer_rsrc((void *)(og + (size_t)tc * ldv), 0, nrow * ldv * 2, kWsBuf);
            u32x4 orw[NHS];  // output-gate inputs: value columns 32 m + 8 g4 .. +8
#pragma unroll
            for (int m = 0; m < NHS; ++m)
                orw[m] = __builtin_amdgcn_raw_buffer_load_b128(ro, 2u * (unsigned)(irow * ldv + 32 * m + 8 * g4), 0, 0);
            if (more && wave == GW) load_gates(c + 1);
            // S^T tiles (jt, it) for jt <= it, k-step outermost so each Q
            // fragment serves all of them; each K fragment is refilled for the
            // next k-step right after its MFMA
            // q.n' of the tile's tokens rides along: an MFMA with n' (high part
            // and remainder) in every row of the A operand
            f32x4 St[NT], qd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jt = 0; jt < NT; ++jt) St[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const bf16 *qrow = Qs + 16 * it * DKP;
            const bf16 *K = Ks[c & 1];
            bf16x8 fq = qk_frag(qrow, 0), fk[NT];
#pragma unroll
            for (int jt = 0; jt < NT; ++jt)
                if (jt <= it) fk[jt] = qk_frag(K + 16 * jt * DKP, 0);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                bf16x8 fqn;
                if (ks + 1 < NKS) fqn = qk_frag(qrow, ks + 1);
                const bf16x8 nh = *reinterpret_cast<const bf16x8 *>(&nhl[c & 1][0][32 * ks + 8 * g4]);
                const bf16x8 nl = *reinterpret_cast<const bf16x8 *>(&nhl[c & 1][1][32 * ks + 8 * g4]);
#pragma unroll
                for (int jt = 0; jt < NT; ++jt) {
                    if (jt <= it) {
                        St[jt] = mfma(fk[jt], fq, St[jt]);
                        if (ks + 1 < NKS) fk[jt] = qk_frag(K + 16 * jt * DKP, ks + 1);
                    }
                }
                qd = mfma(nh, fq, qd);
                qd = mfma(nl, fq, qd);
                if (ks + 1 < NKS) fq = fqn;
            }
            const float qn = qd[0];  // q.n' of token irow
            // P = S (x) e^{u_j - r_i} (j <= i), bf16, in the k order of the V^T fragments
            bf16x4 Pb[NT];
            float rowsum = 0.0f;
            const float ri = G[LP + irow];
#pragma unroll
            for (int jt = 0; jt < NT; ++jt) {
                if (jt <= it) {
                    const f32x4 u4 = *reinterpret_cast<const f32x4 *>(&G[16 * jt + 4 * g4]);
                    float pv[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * jt + 4 * g4 + r;
                        pv[r] = (j <= irow) ? St[jt][r] * __builtin_amdgcn_exp2f(u4[r] - ri) : 0.0f;
                    }
                    rowsum += (pv[0] + pv[1]) + (pv[2] + pv[3]);
                    Pb[jt] = bf16x4{(bf16)pv[0], (bf16)pv[1], (bf16)pv[2], (bf16)pv[3]};
                } else {
                    Pb[jt] = bf16x4{(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
                }
            }
            rowsum += __shfl_xor(rowsum, 16, 64);
            rowsum += __shfl_xor(rowsum, 32, 64);
            if (more && wave == GW) gate_prep(m_next, Gnext);
            // the output-gate loads (and the V copy before them) complete here,
            // before the K copy goes out (the opaque use keeps the compiler from
            // waiting for them later, together with the copies)
#pragma unroll
            for (int m = 0; m < NHS; ++m)
                asm volatile("" : "+v"(orw[m]));
            if (more) copy_tile(Ks[(c + 1) & 1], kg, ldq, QGc{}, tc + L, qko);
            // (X) V(c) landed (only the K copy may stay in flight)
            if (more)
                role_sync<NKS>();
            else
                role_sync<0>();
            if (more) copy_tile(Qs, qg, ldq, QGc{}, tc + L, qko);  // every reader of Q(c) is past X

            // ---- phase 2: O^T of this token tile = scaled read-out + V^T P^T; h
            int vpo[NHS][2];  // V^T fragment offsets by (column tile / 2, read)
#pragma unroll
            for (int m = 0; m < NHS; ++m) {
                vpo[m][0] = vtr_off(prow0, m, tq);
                vpo[m][1] = vtr_off(prow1, m, tq);
            }
            f32x4 acc[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) acc[ct] = Xch[it][ct][lane];
#pragma unroll
            for (int js = 0; js < L / 32; ++js) {
                if (2 * js <= it) {
                    const bf16x8 bp = cat8(Pb[2 * js], Pb[2 * js + 1]);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        const bf16 *vb = Vs + 32 * js * BV + 4 * (ct & 1);
                        const bf16x8 av = cat8(tr_read(vb + vpo[ct >> 1][0]), tr_read(vb + vpo[ct >> 1][1]));
                        acc[ct] = mfma(av, bp, acc[ct]);
                    }
                }
            }
            // token index from an opaque copy of the lane (cheaper to recompute
            // than to keep in a register across the chunk loop)
            int ln2 = lane;
            asm volatile("" : "+v"(ln2));
            const int irow2 = 16 * it + (ln2 & 15);
            // h = a sigmoid(o~) / d = a / (d + d e^{-o~}): one reciprocal per value
            const float den = G[2 * LP + irow2] * qn + rowsum;
            const float dd = fmaxf(fabsf(den), G[3 * LP + irow2]);
            const auto rh = __builtin_amdgcn_make_buffer_rsrc((void *)(hg + (size_t)tc * dv), 0, nrow * dv * 2, kWsBuf);
#pragma unroll
            for (int m = 0; m < NHS; ++m) {
                bf16x8 hv;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const unsigned u = orw[m][e >> 1];
                    const float ox = __uint_as_float((e & 1) ? (u & 0xffff0000u) : (u << 16));
                    const float a = acc[2 * m + (e >> 2)][e & 3];
                    hv[e] = (bf16)(a * __builtin_amdgcn_rcpf(fmaf(dd, exp_e(-ox), dd)));
                }
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hv), rh,
                                                       2u * (unsigned)(irow2 * dv + 32 * m + 8 * g4), 0, 0);
            }
            // (Y) K(c+1), Q(c+1) landed (only this chunk's NHS h stores may stay in flight)
            if (more)
                role_sync<NHS>();
            else
                role_sync<0>();
        }
    }
}

}  // namespace mlstm
