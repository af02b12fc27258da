// chunked.hip -- chunked prefill of the gated delta rule with a per-channel
// gate (Kimi Delta Attention) on gfx950 MFMA.
//
// Recurrence (per sequence and head, "Super Apriel: One Checkpoint, Many
// Speeds", gist.science summary 2a):
//     S_t = S_{t-1} Diag(a_t)(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
//     o_t = scale * S_t q_t.
//
// Chunked form used here (an exact reorganisation; derivation below).  For a
// chunk of C = 64 tokens starting from state S0 (Dv x Dk), with the
// in-chunk cumulative log gate b_r = sum_{s<=r} g_s (per key channel):
//     A[r][s] = sum_j k_rj k_sj e^{b_rj - b_sj}  (s < r)
//     P[r][s] = sum_j q_rj k_sj e^{b_rj - b_sj}  (s <= r)         (C x C)
//     T  = (I + diag(beta) A)^{-1} diag(beta)             (UT transform)
//     X  = V - Kt S0^T,   U = T X,   Kt = k (.) e^{b}     (C x Dv)
//     O  = scale (Qt S0^T + P U),    Qt = q (.) e^{b}
//     S_C = S0 Diag(e^{b_C}) + U^T Kh,   Kh = k (.) e^{b_C - b}
// Derivation: with u_r = beta_r (v_r - S_{r-1} Diag(a_r) k_r) the recurrence
// is S_r = S_{r-1} Diag(a_r) + u_r k_r^T, so S_r = S0 Gamma_r
// + sum_{s<=r} u_s (k_s (.) e^{b_r - b_s})^T with Gamma_r = Diag(e^{b_r}).
// Substituting into u_r gives (I + diag(beta) A) U = diag(beta)(V - Kt S0^T);
// o_r = S_r q_r gives O; S_C is the r = C case.  (The scalar gate takes the
// two-kernel path of chunked_chain.hip.)
//
// Range.  The gate may be anything in [0, 1] (g in [-inf, 0]); g is first
// raised to kGateFloor, which keeps every prefix sum finite.  A chunk whose
// decay stays within e^{kChunkDecayMax} in every channel is factored from
// its first row as above: Kt = k (.) e^{b} and Kb = k (.) e^{-b} stay within
// the range of bf16 and fp32, and A = strict_lower(Kt Kb^T),
// P = lower(Qt Kb^T), Kh = Kb (.) e^{b_C}.  A chunk that decays further in
// some channel ("wide") never forms a factor larger than 1 from the chunk's
// whole decay: with R_I the prefix sum at the end of 16-row block I - 1
// (R_0 = 0, R_4 = b_C),
//     QR = q (.) e^{b - R_I},  KR = k (.) e^{b - R_I}    (rows of block I)
//     KE = k (.) e^{R_{I+1} - b}                          (rows of block I)
// are all at most 1, and every product above is assembled from them:
//     A_IJ = KR_I (KE_J (.) e^{R_I - R_{J+1}})^T          (I > J, factor <= 1)
//     A_II = KR_I (KE_I (.) e^{R_I - R_{I+1}})^T          (factor >= 1)
//     Kt S0^T = KR_I (S0 Diag(e^{R_I}))^T,   Kh_J = KE_J (.) e^{b_C - R_{J+1}}
// The one factor above 1 is the decay of a single 16-row block.  Where some
// channel's block decays by more than e^{kDiagDecayMax}, that diagonal block
// of A and P is formed entry by entry instead, sum_j k_rj k_sj e^{c_rj - c_sj}
// with c the prefix sums within the block (slow_diag below).
//
// Work split.  One workgroup (8 waves) owns one (sequence, head, 32-wide
// slice of Dv) and walks its chunks in order; rows of S never mix, so the
// Dv slices of a head are independent.  The slices of one head run on one
// XCD so their shared reads of q, k and g hit the same L2.  Each chunk:
//   1  prefix sums of the gate logs (two chunks ahead) and the gated
//      operands (one chunk ahead, in registers)
//   2  A (for L = diag(beta) A) and P by 16x16 blocks on MFMA; the four
//      diagonal blocks of (I + L)^{-1} by doubling on 16x16x16 MFMAs
//   3  wave 0: the off-diagonal blocks of T = (I + L)^{-1} diag(beta) by
//      16x16x16 MFMA block substitution; waves 4-7: X = V - Kt S0^T and
//      Qt S0^T on MFMA
//   4  U = T X
//   5  O = Qt S0^T + P U, and S^T <- e^{b_C} (.) S^T + Kh^T U
// All contractions use bf16 operands with fp32 accumulation; the state is
// carried in fp32 registers and rounded to bf16 only as an MFMA operand.
//
// Gate layout.  Lane l of wave w holds rows RPT (w RPW + l % RPW) .. +RPT-1
// of key channels 8 (l / RPW) .. +7 (CG = D/8 channel groups, RPW = 64/CG row
// groups per wave), so each load instruction reads whole rows; the prefix
// sums over rows run inside the wave across the RPW adjacent lanes of a
// channel group (DPP), then across the waves through per-wave totals in LDS
// that two waves turn into prefixes.
#include <type_traits>

#include "gdr_internal.h"
#include "device_util.h"

namespace gdr {
namespace {

constexpr int C = 64;       // chunk length
constexpr int NW = 8;       // waves per workgroup
constexpr int NT = NW * 64; // threads per workgroup
constexpr int BV = 32;      // value columns per workgroup
constexpr int PC = C + 8;   // padded LDS row length for C-wide bf16 rows
constexpr int PCT = C + 16; // C-wide bf16 rows read by transpose loads: a row
                            // stride of 40 dwords puts 4 consecutive rows on
                            // disjoint banks
constexpr int PY = 24;      // padded row length of the bf16 Y^T blocks (read by
                            // transpose loads: 4 consecutive rows on disjoint banks)
constexpr int PV = BV + 8;  // padded LDS row length of the v tile
// A chunk whose summed log-decay exceeds kChunkDecayMax in some channel
// takes the block-reference form; in it, a 16-row diagonal block whose
// summed log-decay exceeds kDiagDecayMax in some channel takes the
// entry-by-entry form.  Below these, the factors stay under e^80 (e^70) and
// their partners above e^-80 (e^-70) times k, inside the normal range.
constexpr float kChunkDecayMax = 80.f;
constexpr float kDiagDecayMax = 70.f;
// flag bits of a chunk: 0..3 diagonal blocks formed entry by entry, 4 wide
constexpr int kWide = 16;

// Per-thread indices used by every phase.
template <int D> struct LaneIds {
    static constexpr int CG = D / 8;           // 8-channel groups per row
    static constexpr int RPW = 64 / CG;        // row groups per wave
    static constexpr int RPT = C / (NW * RPW); // rows per thread in the gate phase
    int tid, lane, w, l15, l4;
    int cg, rgl, rg;   // gate phase: channel group, row group in the wave / block
    int vr, vc;        // v tile: row, first column
    __device__ explicit LaneIds(int t) {
        tid = t;
        lane = t & 63;
        w = __builtin_amdgcn_readfirstlane(t >> 6);
        l15 = lane & 15;
        l4 = lane >> 4;
        cg = lane / RPW;
        rgl = lane % RPW;
        rg = w * RPW + rgl;
        vr = t >> 3;
        vc = (t & 7) * 4;
    }
};

// Inclusive prefix sum over the RPW (4 or 8) adjacent lanes of each group:
// two quad permutes within the quad, then for RPW = 8 the last lane of the
// lower quad added to the upper quad (quad broadcast, row_shr:4).
template <int RPW>
__device__ inline float group_scan(float x, int lane) {
    auto dpp = [](float v, auto ctrl) -> float {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                     decltype(ctrl)::value, 0xF, 0xF, true));
    };
    const int q = lane & 3;
    float y = dpp(x, std::integral_constant<int, 0x90>{});   // quad_perm [0,0,1,2]
    x += q >= 1 ? y : 0.f;
    y = dpp(x, std::integral_constant<int, 0x40>{});         // quad_perm [0,0,0,1]
    x += q >= 2 ? y : 0.f;
    if (RPW == 8) {
        y = dpp(dpp(x, std::integral_constant<int, 0xFF>{}),  // quad_perm [3,3,3,3]
                std::integral_constant<int, 0x114>{});        // row_shr:4
        x += (lane & 4) ? y : 0.f;
    }
    return x;
}

template <int D> struct Smem {
    static constexpr int PD = D + 8;   // padded row length for D-wide rows
    alignas(16) bf16 Q[C * PD];        // QR = q (.) e^{b - R_I}, [r][j]
    alignas(16) bf16 K[C * PD];        // KR = k (.) e^{b - R_I}, [r][j]
    alignas(16) bf16 Kb[2][C * PD];    // KE = k (.) e^{R_{I+1} - b}, [r][j], by chunk parity
    alignas(16) bf16 S[BV * PD];       // bf16 copy of the state slice, [i][j]
    alignas(16) bf16 TT[C * PCT];      // T^T, [s][r] (read back by transpose loads)
    alignas(16) bf16 PT[C * PCT];      // P^T, [s][r]
    alignas(16) bf16 XT[BV * PC];      // X^T, [i][s]
    alignas(16) bf16 UT[BV * PC];      // U^T, [i][s]
    alignas(16) bf16 V[C * PV];        // v tile, [r][i]
    alignas(16) bf16 LTo[6][16 * PY];  // blocks (I > J) of L^T = (diag(beta) A)^T, [ltri(I, J)][s][r]
    alignas(16) bf16 YT[4 * 16 * PY];  // inverted diagonal blocks, transposed: [b][c][r]
    alignas(16) float QS[8 * 64 * 4];  // Qt S0^T of the prep chunk, transposed, in
                                       // accumulator order: [4 jv + I][lane][e]
    alignas(16) float beta[C];
    alignas(16) float gam[2][D];       // e^{b_C} per channel, by chunk parity
    // per-channel factors of a chunk, from its block ends R_1..R_3 and b_C:
    //   FD (prep chunk only): e^{R_b - R_{b+1}}, b = 0..3, then e^{R_2 - R_1},
    //      e^{R_3 - R_1}, e^{R_3 - R_2} for the blocks (2,0), (3,0), (3,1)
    //   FX (by parity): e^{R_1}, e^{R_2}, e^{R_3}
    //   FU (by parity): e^{b_C - R_1}, e^{b_C - R_2}, e^{b_C - R_3}
    alignas(16) float FD[7][D];
    alignas(16) float FX[2][3][D];
    alignas(16) float FU[2][3][D];
    // A (0) and P (1) of the diagonal blocks formed entry by entry, [b][r][s]
    alignas(16) float dres[2][4][256];
    alignas(16) float rnorm[2][2][C];  // RAW: 1/|q_r|, 1/|k_r| by chunk parity
    int dflag[2][2];                   // reference pass, by chunk parity: per-wave parts of
                                       // the chunk's diagonal blocks to form entry by entry
    int wide_any;                      // plain pass: some chunk so far is wide
    // per chunk parity: the per-wave sums of the gate logs [w][j], turned in
    // place into their exclusive prefix over the waves, and the chunk total
    // b_C in row NW, all times log2(e)
    alignas(16) float pfx[2][(NW + 1) * D];
};


// Software pipeline.  Iteration j of the chunk loop works on four chunks at
// once, with three workgroup barriers:
//   chunk j-1 ("state"):  U = T X, then O = Qt S0^T + P U and the state update
//   chunk j   ("prep"):   gated operands -> LDS, A -> L, T (diagonal blocks by
//                         doubling, the rest by block substitution), P,
//                         X, Qt S0^T
//   chunk j+1 ("gate"):   gated operands in registers
//   chunk j+2 ("scan"):   prefix sums of the gate logs
//   phase A: U(j-1) (waves 0-3) || store gated operands of chunk j
//   phase B: waves 0-3: the diagonal block (b, b) of A and P, its inverse,
//            block (b, b-1), then O(j-1);  waves 4-7: the state update
//            (j-1), then blocks (2,0), (3,0), (3,1);  all: prefix sums of
//            the gate logs of chunk j+2 within each wave, loads of g(j+3)
//   phase C: T(j) off-diagonal (wave 0) || Qt S0^T(j), X(j) (waves 4-7);
//            all: P(j) -> LDS; waves 1-2: prefixes over the waves for chunk
//            j+2; all: gated operands of chunk j+1, loads of q, k, v(j+2)
// P(j) is held in registers from phase B to phase C because the O of chunk
// j-1 reads the previous P during phase B.
// RAW: raw projections (fused preprocessing).  q and k are normalised at
// gating time (the row norms come from the 16 lanes that hold a row), the
// gate logits are turned into -c softplus at the scan (zero for rows past the
// sequence end, which must not decay the state), beta from its logit when
// staged.
template <int D, bool RAW, bool REF>
__global__ __launch_bounds__(NT, 1) void chunked_kernel(PrefillArgs a) {
    using Sm = Smem<D>;
    using LI = LaneIds<D>;
    constexpr int PD = Sm::PD;
    constexpr int NTILE = D / BV;
    constexpr int RPW = LI::RPW;
    constexpr int RPT = LI::RPT;
    constexpr int KD = D / 32;         // x32 steps over a D-long contraction
    constexpr int SBK = D / 64;        // 16-row blocks of S^T per state wave
    static_assert(RPT >= 1, "gate phase layout");
    __shared__ Sm sm;

    // ---- work mapping: the Dv slices of one (sequence, head) share an XCD
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int jj = bid >> 3;
    const int tile = jj % NTILE;
    const int unit = (jj / NTILE) * 8 + xcd;
    if (unit >= a.N * a.H) return;
    const int rank = unit / a.H;
    const int h = unit - rank * a.H;
    const int n = a.order ? a.order[rank] : rank;
    // the reference pass redoes only the (sequence, head) pairs the plain
    // pass left to it
    if (REF && !a.unit_wide[(size_t)n * a.H + h]) return;
    long long t0, t1;
    if (a.cu_seqlens) {
        t0 = a.cu_seqlens[n];
        t1 = a.cu_seqlens[n + 1];
    } else {
        t0 = (long long)n * a.T;
        t1 = t0 + a.T;
    }
    const int i0 = tile * BV;
    const size_t tokstride = (size_t)a.H * D;
    const bf16 *qg = static_cast<const bf16 *>(a.q) + (size_t)h * D;
    const bf16 *kg = static_cast<const bf16 *>(a.k) + (size_t)h * D;
    const bf16 *vg = static_cast<const bf16 *>(a.v) + (size_t)h * D + i0;
    bf16 *og = static_cast<bf16 *>(a.o) + (size_t)h * D + i0;
    const long long nch = (t1 - t0 + C - 1) / C;
    // first global chunk of the sequence (the index of its states)
    const long long cbase = !a.states ? 0 : a.cu_seqlens ? a.chunk_base[n] : (long long)n * nch;
    const int tid0 = threadIdx.x;

    // T and P are lower triangular: the entries above the diagonal of T^T and
    // P^T stay zero, only lower blocks are ever written
    for (int e = tid0; e < C * PCT; e += NT) {
        sm.TT[e] = (bf16)0.f;
        sm.PT[e] = (bf16)0.f;
    }
    if (tid0 == 0) sm.wide_any = 0;

    // ---- state S^T in registers of waves 4..7: wave w holds blocks
    //      (Jk, Jv) for Jk = SBK*(w-4) + kb, Jv = 0, 1, i.e. S^T[j][iv] with
    //      j = 16*Jk + 4*l4 + e, iv = 16*Jv + l15
    f32x4 St[SBK][2];
    {
        const LI L(tid0);
        const float *h0p = seq_h0<D>(a, n, h);
#pragma unroll
        for (int kb = 0; kb < SBK; ++kb) {
#pragma unroll
            for (int jv = 0; jv < 2; ++jv) {
                f32x4 sv = {0.f, 0.f, 0.f, 0.f};
                if (L.w >= 4) {
                    const int j = 16 * (SBK * (L.w - 4) + kb) + 4 * L.l4;
                    const int iv = 16 * jv + L.l15;
                    if (h0p)
                        sv = *reinterpret_cast<const f32x4 *>(h0p + (size_t)(i0 + iv) * D + j);
                    *reinterpret_cast<bf16x4 *>(&sm.S[iv * PD + j]) = cvt4(sv);
                    if (a.states && nch > 0)        // the state entering chunk 0
                        *reinterpret_cast<f32x4 *>(a.states + ((size_t)cbase * a.H + h) * D * D +
                                                   (size_t)(i0 + iv) * D + j) = sv;
                }
                St[kb][jv] = sv;
            }
        }
    }

    // raw inputs held in registers ahead of use: the gate logs of the chunk
    // to be scanned next (reloaded right after its prefix sums are taken), q
    // and k of the chunk to be gated next (reloaded right after they are
    // gated), and v/beta of the next two chunks (by chunk parity)
    bf16x8 rq[RPT], rk[RPT];
    f32x4 rgc[RPT][2];
    bf16x8 rgx[RPT];                 // RAW: gate logits
    float rgf[RPT][8];               // RAW: their gate logs, -c softplus
    bf16x4 rv[2];
    float rb[2];
    rv[0] = rv[1] = bf16x4{};
    rb[0] = rb[1] = 0.f;
    // rows of chunk c (0 past the end); the extents below cover exactly the
    // valid rows, so loads of rows >= valid_rows(c) return zeros
    auto valid_rows = [&](long long c) -> int {
        const long long rem = t1 - (t0 + c * C);
        return rem <= 0 ? 0 : (rem < C ? (int)rem : C);
    };
    auto load_g = [&](const LI &L, long long c) {
        const long long tc = t0 + c * C;
        const int Cc = valid_rows(c);
        if (RAW) {
            const unsigned rowx = (unsigned)(a.H * D * 2);
            const rsrc_t rs = make_rsrc(static_cast<const bf16 *>(a.xg) + ((size_t)tc * a.H + h) * D,
                                        Cc ? (Cc - 1) * rowx + D * 2 : 0u);
#pragma unroll
            for (int i = 0; i < RPT; ++i) rgx[i] = bload16(rs, (L.rg * RPT + i) * rowx + 16 * L.cg);
            return;
        }
        const unsigned rowb = (unsigned)(a.H * D * 4);
        const rsrc_t rs = make_rsrc(a.g + ((size_t)tc * a.H + h) * D,
                                    Cc ? (Cc - 1) * rowb + D * 4 : 0u);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const unsigned off = (L.rg * RPT + i) * rowb + 32 * L.cg;
            rgc[i][0] = bload16f(rs, off);
            rgc[i][1] = bload16f(rs, off + 16);
        }
    };
    auto load_qkvb = [&](const LI &L, long long c, int par) {
        const long long tc = t0 + c * C;
        const int Cc = valid_rows(c);
        const unsigned rowb = (unsigned)(tokstride * 2);
        const rsrc_t rq_s = make_rsrc(qg + (size_t)tc * tokstride, Cc ? (Cc - 1) * rowb + D * 2 : 0u);
        const rsrc_t rk_s = make_rsrc(kg + (size_t)tc * tokstride, Cc ? (Cc - 1) * rowb + D * 2 : 0u);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const unsigned off = (L.rg * RPT + i) * rowb + 16 * L.cg;
            rq[i] = bload16(rq_s, off);
            rk[i] = bload16(rk_s, off);
        }
        const rsrc_t rv_s = make_rsrc(vg + (size_t)tc * tokstride, Cc ? (Cc - 1) * rowb + BV * 2 : 0u);
        rv[par] = bload8(rv_s, L.vr * rowb + 2 * L.vc);
        if (RAW) {
            const unsigned browx = (unsigned)(a.H * 2);
            const rsrc_t rb_s = make_rsrc(static_cast<const bf16 *>(a.xb) + (size_t)tc * a.H + h,
                                          Cc ? (Cc - 1) * browx + 2 : 0u);
            rb[par] = bf16_bits_to_float(bload2(rb_s, L.tid * browx));
        } else {
            const unsigned browb = (unsigned)(a.H * 4);
            const rsrc_t rb_s = make_rsrc(a.beta + (size_t)tc * a.H + h, Cc ? (Cc - 1) * browb + 4 : 0u);
            rb[par] = bload4(rb_s, L.tid * browb);
        }
    };

    // gated operands Qt, Kt, Kb of the next chunk, held in registers from
    // phase C to the next phase A; prefix sums of the gate logs within the
    // wave for the next two chunks (by chunk parity), held from their scan
    // (phase B, two chunks ahead) to their gating
    bf16x8 gq[RPT], gk[RPT], gkb[RPT];
    float cum[2][RPT][8];
    constexpr float kL2e = 1.4426950408889634f;

    // prefix sums of the gate logs of one chunk over this wave's rows
    // (phase B); the wave's per-channel totals go to pfx[par]
    // RAW: gate logs of chunk c from its logits (zero past the sequence end),
    // a phase ahead of the scan that reads them
    auto softplus_g = [&](const LI &L, long long c) {
        const int Cc = valid_rows(c);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const bool live = L.rg * RPT + i < Cc;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                rgf[i][e] = live ? neg_softplus((float)rgx[i][e], a.gate_scale) : 0.f;
        }
    };
    auto scan = [&](const LI &L, auto par_tag) {
        constexpr int par = decltype(par_tag)::value;
        float run[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) run[e] = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float gv = RAW ? rgf[i][e] : rgc[i][e >> 2][e & 3];
                run[e] += __builtin_fmaxf(gv, kGateFloor);
                cum[par][i][e] = run[e];
            }
        }
        // scan of the row-group totals across the lanes of the channel group
        float incl[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) incl[e] = group_scan<RPW>(run[e], L.lane);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) cum[par][i][e] += incl[e] - run[e];
        }
        if (L.rgl == RPW - 1) {
            float *t = &sm.pfx[par][L.w * D + 8 * L.cg];
            *reinterpret_cast<f32x4 *>(t) = f32x4{incl[0], incl[1], incl[2], incl[3]};
            *reinterpret_cast<f32x4 *>(t + 4) = f32x4{incl[4], incl[5], incl[6], incl[7]};
        }
    };

    // per-wave totals -> exclusive prefix over the waves and chunk total, one
    // thread per key channel (threads 64 .. 64+D-1, phase C); and flags:
    // the plain pass notes a chunk that some channel decays by more than
    // e^{kChunkDecayMax} over the chunk (wide), the reference pass the 16-row blocks
    // (two waves each) that some channel decays by more than e^{kDiagDecayMax}
    auto prefix = [&](int par) {
        const int ch = tid0 - 64;
        int fl = 0;
        if (ch >= 0 && ch < D) {
            float t[NW];
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) t[ww] = sm.pfx[par][ww * D + ch];
            float acc = 0.f, rb = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                sm.pfx[par][ww * D + ch] = acc * kL2e;
                acc += t[ww];
                if (REF && (ww & 1)) {
                    if (rb - acc > kDiagDecayMax) fl |= 1 << (ww >> 1);
                    rb = acc;
                }
            }
            sm.pfx[par][NW * D + ch] = acc * kL2e;
            if (!REF && !(-acc <= kChunkDecayMax)) fl = kWide;
        }
        const int wv = __builtin_amdgcn_readfirstlane(tid0 >> 6);
        if (wv == 1 || wv == 2) {
            if (REF) {
                int m = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    if (__ballot((fl >> b) & 1)) m |= 1 << b;
                if ((tid0 & 63) == 0) sm.dflag[par][wv - 1] = m;
            } else if (__ballot(fl != 0) && (tid0 & 63) == 0) {
                sm.wide_any = 1;
            }
        }
    };
    // reference pass: the diagonal blocks to form entry by entry of the
    // chunk whose prefix sums are in pfx[par], wave-uniform
    auto chunk_flags = [&](int par) -> int {
        return __builtin_amdgcn_readfirstlane(sm.dflag[par][0] | sm.dflag[par][1]);
    };

    // gated operands of one chunk (phase C) into registers: Qt, Kt, Kb, or
    // for a wide chunk QR, KR, KE (the same formulas with the references
    // R_I, R_{I+1} in place of 0); e^{b_C}, for a wide chunk the factors,
    // and (RAW) the row norms into their buffers
    auto gate = [&](const LI &L, auto par_tag) {
        constexpr int par = decltype(par_tag)::value;
        constexpr bool wide = REF;
        auto ld8f = [&](int row, float (&v)[8]) {
            const float *p = &sm.pfx[par][row * D + 8 * L.cg];
            const f32x4 x0 = *reinterpret_cast<const f32x4 *>(p);
            const f32x4 x1 = *reinterpret_cast<const f32x4 *>(p + 4);
            v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
            v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
        };
        const int Ib = L.w >> 1;             // this wave's 16-row block
        float pre[8], r0[8] = {}, r1[8] = {};
        ld8f(L.w, pre);                      // prefix sum before this wave's rows
        if (wide) {
            ld8f(2 * Ib, r0);                // R_I
            ld8f(2 * Ib + 2, r1);            // R_{I+1} (b_C for the last block)
        }
        if (wide) {
            // the chunk's per-channel factors: NT / D threads per channel,
            // 14 vectors between them
            constexpr int G = NT / D;
            const int ch = L.tid % D, grp = L.tid / D;
            const float *pf = sm.pfx[par];
            const float R1 = pf[2 * D + ch], R2 = pf[4 * D + ch], R3 = pf[6 * D + ch],
                        bC = pf[NW * D + ch];
#pragma unroll
            for (int v = 0; v < 14; ++v) {
                if (v % G != grp) continue;
                float x;
                float *dst;
                switch (v) {
                case 0: x = -R1; dst = &sm.FD[0][ch]; break;
                case 1: x = R1 - R2; dst = &sm.FD[1][ch]; break;
                case 2: x = R2 - R3; dst = &sm.FD[2][ch]; break;
                case 3: x = R3 - bC; dst = &sm.FD[3][ch]; break;
                case 4: x = R2 - R1; dst = &sm.FD[4][ch]; break;
                case 5: x = R3 - R1; dst = &sm.FD[5][ch]; break;
                case 6: x = R3 - R2; dst = &sm.FD[6][ch]; break;
                case 7: x = R1; dst = &sm.FX[par][0][ch]; break;
                case 8: x = R2; dst = &sm.FX[par][1][ch]; break;
                case 9: x = R3; dst = &sm.FX[par][2][ch]; break;
                case 10: x = bC - R1; dst = &sm.FU[par][0][ch]; break;
                case 11: x = bC - R2; dst = &sm.FU[par][1][ch]; break;
                case 12: x = bC - R3; dst = &sm.FU[par][2][ch]; break;
                default: x = bC; dst = &sm.gam[par][ch]; break;
                }
                *dst = __builtin_amdgcn_exp2f(x);
            }
        } else if (L.rg == 0) {
            float bC[8], gC[8];
            ld8f(NW, bC);
#pragma unroll
            for (int e = 0; e < 8; ++e) gC[e] = __builtin_amdgcn_exp2f(bC[e]);
            *reinterpret_cast<f32x4 *>(&sm.gam[par][8 * L.cg]) = f32x4{gC[0], gC[1], gC[2], gC[3]};
            *reinterpret_cast<f32x4 *>(&sm.gam[par][8 * L.cg + 4]) = f32x4{gC[4], gC[5], gC[6], gC[7]};
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            float qt[8], kt[8], kb[8];
            float nq = 1.f, nk = 1.f;
            if (RAW) {
                // |q_r|^2, |k_r|^2 over the CG lanes holding row r (lanes
                // rgl + RPW m)
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sq = __builtin_fmaf((float)rq[i][e], (float)rq[i][e], sq);
                    sk = __builtin_fmaf((float)rk[i][e], (float)rk[i][e], sk);
                }
                sq = sum_stride<RPW>(sq);
                sk = sum_stride<RPW>(sk);
                nq = inv_norm(sq);
                nk = inv_norm(sk);
                if (L.cg == 0) {
                    sm.rnorm[par][0][L.rg * RPT + i] = nq;
                    sm.rnorm[par][1][L.rg * RPT + i] = nk;
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float b2 = __builtin_fmaf(cum[par][i][e], kL2e, pre[e]);
                float er, ee;
                if (REF) {
                    er = __builtin_amdgcn_exp2f(b2 - r0[e]);          // e^{b - R_I}
                    ee = __builtin_amdgcn_exp2f(r1[e] - b2);          // e^{R_{I+1} - b}
                } else {
                    er = __builtin_amdgcn_exp2f(b2);                  // e^{b}
                    ee = __builtin_amdgcn_rcpf(er);                   // e^{-b}
                }
                const float kv = RAW ? (float)rk[i][e] * nk : (float)rk[i][e];
                qt[e] = (RAW ? (float)rq[i][e] * nq : (float)rq[i][e]) * er;
                kt[e] = kv * er;
                kb[e] = kv * ee;
            }
            gq[i] = cvt8(qt);
            gk[i] = cvt8(kt);
            gkb[i] = cvt8(kb);
        }
    };

    // gated operands, v tile and beta of one chunk into LDS (phase A)
    auto store_gate = [&](const LI &L, int par) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const unsigned e = (unsigned)((L.rg * RPT + i) * PD + 8 * L.cg);
            *reinterpret_cast<bf16x8 *>(sm.Q + e) = gq[i];
            *reinterpret_cast<bf16x8 *>(sm.K + e) = gk[i];
            *reinterpret_cast<bf16x8 *>(sm.Kb[par] + e) = gkb[i];
        }
        *reinterpret_cast<bf16x4 *>(sm.V + (unsigned)(L.vr * PV + L.vc)) = rv[par];
        if (L.tid < C) sm.beta[L.tid] = RAW ? logistic(rb[par]) : rb[par];
    };

    // Diagonal 16x16 blocks of A and P entry by entry, for the blocks of
    // chunk j set in fl (all threads, a block at a time; ends with a
    // barrier):  A[r][s] = sum_j k_rj k_sj 2^{c_rj - c_sj} (s < r) and
    // P[r][s] = sum_j q_rj k_sj 2^{c_rj - c_sj} (s <= r), with c the prefix
    // sums of the block's gate logs (log2 units), so every factor is at most
    // 1 whatever the decay.  The block's rows of g, k and q come from global
    // memory into buffers that are free at this point: c in TT, k in XT, q
    // in LTo (TT is zeroed again afterwards, as its upper blocks must stay
    // zero).  Four threads share a pair (r, s), a quarter of the channels
    // each.
    auto slow_diag = [&](const LI &L, long long j, int fl, int par) {
        float *cs = reinterpret_cast<float *>(sm.TT);
        bf16 *ks = sm.XT;
        bf16 *qs = &sm.LTo[0][0];
        static_assert(16 * D * 4 <= sizeof(sm.TT) && 16 * D * 2 <= sizeof(sm.XT) &&
                      16 * D * 2 <= sizeof(sm.LTo), "entry-by-entry scratch");
        const long long tc = t0 + j * C;
        const int Cc = valid_rows(j);
        const unsigned rowb = (unsigned)(tokstride * 2);
        for (int b = 0; b < 4; ++b) {
            if (!((fl >> b) & 1)) continue;
            const int nr = Cc - 16 * b <= 0 ? 0 : (Cc - 16 * b > 16 ? 16 : Cc - 16 * b);
            const size_t tb = (size_t)(tc + 16 * b);   // first token of the block
            if (L.tid < D) {
                const int ch = L.tid;
                const unsigned rowx = (unsigned)(a.H * D * (RAW ? 2 : 4));
                const rsrc_t rs = RAW ? make_rsrc(static_cast<const bf16 *>(a.xg) + (tb * a.H + h) * D,
                                                  nr ? (nr - 1) * rowx + D * 2 : 0u)
                                      : make_rsrc(a.g + (tb * a.H + h) * D, nr ? (nr - 1) * rowx + D * 4 : 0u);
                float run = 0.f;
#pragma unroll 1
                for (int r4 = 0; r4 < 16; r4 += 4) {
                    float gv[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int r = r4 + u;
                        if (RAW) {
                            const float x = bf16_bits_to_float(bload2(rs, r * rowx + 2 * ch));
                            gv[u] = r < nr ? neg_softplus(x, a.gate_scale) : 0.f;
                        } else {
                            gv[u] = bload4(rs, r * rowx + 4 * ch);
                        }
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        run += __builtin_fmaxf(gv[u], kGateFloor);
                        cs[(r4 + u) * D + ch] = run * kL2e;
                    }
                }
            }
            constexpr int NP = 16 * D / 8;           // 16-byte pieces of a block of rows
            const rsrc_t rkb = make_rsrc(kg + tb * tokstride, nr ? (nr - 1) * rowb + D * 2 : 0u);
            const rsrc_t rqb = make_rsrc(qg + tb * tokstride, nr ? (nr - 1) * rowb + D * 2 : 0u);
            for (int p = L.tid; p < 2 * NP; p += NT) {
                const int which = __builtin_amdgcn_readfirstlane(p / NP);   // whole waves
                const int pp = p % NP, r = pp / (D / 8), c8 = pp % (D / 8);
                const bf16x8 v = bload16(which ? rqb : rkb, r * rowb + 16 * c8);
                *reinterpret_cast<bf16x8 *>((which ? qs : ks) + r * D + 8 * c8) = v;
            }
            __syncthreads();
            for (int p = L.tid >> 2; p < 136; p += NT / 4) {
                int r = 0;
                while ((r + 1) * (r + 2) / 2 <= p) ++r;
                const int s2 = p - r * (r + 1) / 2;
                const int qq = L.tid & 3;
                float aa = 0.f, pp = 0.f;
#pragma unroll 2
                for (int u = 0; u < D / 4; ++u) {
                    const int ch = 4 * u + qq;
                    const float e = __builtin_amdgcn_exp2f(cs[r * D + ch] - cs[s2 * D + ch]);
                    const float kse = (float)ks[s2 * D + ch] * e;
                    aa = __builtin_fmaf((float)ks[r * D + ch], kse, aa);
                    pp = __builtin_fmaf((float)qs[r * D + ch], kse, pp);
                }
                aa += dpp_f<0xB1>(aa);
                aa += dpp_f<0x4E>(aa);
                pp += dpp_f<0xB1>(pp);
                pp += dpp_f<0x4E>(pp);
                if (qq == 0) {
                    if (RAW) {
                        const float nks = sm.rnorm[par][1][16 * b + s2];
                        aa *= sm.rnorm[par][1][16 * b + r] * nks;
                        pp *= sm.rnorm[par][0][16 * b + r] * nks;
                    }
                    sm.dres[0][b][r * 16 + s2] = aa;
                    sm.dres[1][b][r * 16 + s2] = pp;
                }
            }
            __syncthreads();
        }
        for (int e = L.tid; e < C * PCT; e += NT) sm.TT[e] = (bf16)0.f;
        __syncthreads();
    };

    // ---- one pipeline iteration; PAR = parity of the prep chunk j
    auto iteration = [&](auto par_tag, auto s_tag, auto p_tag, long long j) {
        constexpr int PAR = decltype(par_tag)::value;
        const LI L(opaque(tid0));
        const int lane = L.lane, w = L.w, l15 = L.l15, l4 = L.l4;
        constexpr bool hasS = decltype(s_tag)::value;   // j >= 1
        constexpr bool hasP = decltype(p_tag)::value;   // j < nch
        const bool hasG = j + 1 < nch;

        // fragment entries times per-channel factors f_j (LDS), for the
        // channels a fragment lane holds (32 kk + 8 (lane >> 4) .. +7)
        auto scale_frag = [&](bf16x8 &fr, int kk, const float *f) {
            const int c0 = 32 * kk + 8 * (lane >> 4);
            const f32x4 f0 = *reinterpret_cast<const f32x4 *>(f + c0);
            const f32x4 f1 = *reinterpret_cast<const f32x4 *>(f + c0 + 4);
#pragma unroll
            for (int u = 0; u < 8; ++u) fr[u] = (bf16)((float)fr[u] * (u < 4 ? f0[u] : f1[u - 4]));
        };
        auto frags = [&](const bf16 *M, int blk, bf16x8 (&f)[KD]) {
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) f[kk] = frag_rows(M, PD, 16 * blk, 32 * kk, lane);
        };
        // A and P block (I, J): KR and QR rows of block I against KE rows of J
        // (their fragments kf, qf, bf)
        auto gram = [&](const bf16x8 (&kf)[KD], const bf16x8 (&qf)[KD], const bf16x8 (&bf)[KD],
                        f32x4 &av, f32x4 &pv) {
            av = f32x4{0.f, 0.f, 0.f, 0.f};
            pv = av;
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) {
                av = mfma32(kf[kk], bf[kk], av);
                pv = mfma32(qf[kk], bf[kk], pv);
            }
        };
        // L^T[s][r] = beta_r A[r][s] of a block below the diagonal (I > J)
        auto putL = [&](int I, int J, f32x4 av) {
            const int r0 = 16 * I + 4 * l4;
            const f32x4 br = *reinterpret_cast<const f32x4 *>(&sm.beta[r0]);
            *reinterpret_cast<bf16x4 *>(&sm.LTo[I * (I - 1) / 2 + J][l15 * PY + 4 * l4]) = cvt4(av * br);
        };
        // P^T[s][r] = P[r][s] for s <= r
        auto putP = [&](int I, int J, f32x4 pv) {
            const int s = 16 * J + l15;
            const int r0 = 16 * I + 4 * l4;
            f32x4 pm;
#pragma unroll
            for (int e = 0; e < 4; ++e) pm[e] = s <= r0 + e ? pv[e] : 0.f;
            *reinterpret_cast<bf16x4 *>(&sm.PT[s * PCT + r0]) = cvt4(pm);
        };
        // P blocks of chunk j computed in phase B, written in phase C
        f32x4 pdiag = {0.f, 0.f, 0.f, 0.f}, poff = pdiag;

        // reference pass: the diagonal blocks of chunk j to form entry by
        // entry (read now, used after phase A)
        const int flP = (REF && hasP) ? chunk_flags(PAR) : 0;

        // ================= phase A ========================================
        if (hasS && w < 4) {   // U = T X of chunk j-1; wave w: row block w
            const int I = w;
            const bf16x8 t0f = frag_cols(sm.TT, PCT, 0, 16 * I, lane);
            bf16x8 t1f = {};
            if (I >= 2) t1f = frag_cols(sm.TT, PCT, 32, 16 * I, lane);
#pragma unroll
            for (int jv = 0; jv < 2; ++jv) {
                f32x4 u = mfma32(t0f, frag_rows(sm.XT, PC, 16 * jv, 0, lane), f32x4{0.f, 0.f, 0.f, 0.f});
                if (I >= 2)   // T is lower triangular: rows < 32 need s < 32 only
                    u = mfma32(t1f, frag_rows(sm.XT, PC, 16 * jv, 32, lane), u);
                *reinterpret_cast<bf16x4 *>(&sm.UT[(16 * jv + l15) * PC + 16 * I + 4 * l4]) = cvt4(u);
            }
        }
        if (hasP) store_gate(L, PAR);
        if (RAW && j + 2 < nch) softplus_g(L, j + 2);
        __syncthreads();

        // ================= phase B ========================================
        // diagonal blocks of a wide chunk that decay too fast for the
        // reference of their first row: entry by entry, before the rest of
        // the phase
        if (REF && flP) slow_diag(L, j, flP, PAR);
        if (w < 4) {
            if (hasP) {
                // diagonal block (b, b) and, for b >= 1, block (b, b-1): the
                // latter's products run while the diagonal block is inverted
                const int b = w;
                bf16x8 kf[KD], qf[KD], bf[KD];
                frags(sm.K, b, kf);
                frags(sm.Q, b, qf);
                f32x4 ad, adT = {0.f, 0.f, 0.f, 0.f};
                if (REF && ((flP >> b) & 1)) {
                    const float *Ar = sm.dres[0][b], *Pr = sm.dres[1][b];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ad[e] = Ar[(4 * l4 + e) * 16 + l15];
                        adT[e] = Ar[l15 * 16 + 4 * l4 + e];
                        pdiag[e] = Pr[(4 * l4 + e) * 16 + l15];
                    }
                } else {
                    // wide: against KE_b (.) e^{R_b - R_{b+1}} (at most e^{kDiagDecayMax})
                    frags(sm.Kb[PAR], b, bf);
                    if (REF) {
#pragma unroll
                        for (int kk = 0; kk < KD; ++kk) scale_frag(bf[kk], kk, sm.FD[b]);
                    }
                    gram(kf, qf, bf, ad, pdiag);
#pragma unroll
                    for (int kk = 0; kk < KD; ++kk) adT = mfma32(bf[kk], kf[kk], adT);   // A_bb^T
                }
                f32x4 aoff = {0.f, 0.f, 0.f, 0.f};
                if (b >= 1) {
                    frags(sm.Kb[PAR], b - 1, bf);
                    gram(kf, qf, bf, aoff, poff);
                }
                // M = L_bb = strict_lower(diag(beta) A_bb) as acc(M) and
                // acc(M^T) (lane holds M[4 l4 + e][l15], M^T[4 l4 + e][l15]).
                // Y = (I + M)^{-1} by doubling: with Y_k the inverse of the
                // part of I + M inside the diagonal blocks of size 2^k and E_k
                // the part of M joining the two halves of each block of size
                // 2^{k+1}, Y_{k+1} = Y_k - Y_k E_k Y_k exactly (E_k Y_k E_k = 0),
                // from Y_0 = I to Y_4 = Y.  Every term is an entry of a true
                // inverse times entries of M, so the bf16 operands never carry
                // the large, cancelling terms of a power series in M.  An
                // MFMA with A operand acc(X^T) and B operand acc(Z) yields
                // acc(X Z); Y and Y^T are carried side by side.
                const float bl = sm.beta[16 * b + l15];
                const f32x4 br4 = *reinterpret_cast<const f32x4 *>(&sm.beta[16 * b + 4 * l4]);
                f32x4 MT, Mn;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int sl = 4 * l4 + e;
                    MT[e] = sl < l15 ? bl * adT[e] : 0.f;
                    Mn[e] = sl > l15 ? br4[e] * ad[e] : 0.f;
                }
                // entry (r, s) of E_k: r, s in one block of 2^{k+1}, r in its
                // lower and s in its upper half
                auto joins = [](int k, int r, int sc) {
                    return (r >> k) == (sc >> k) + 1 && (r >> (k + 1)) == (sc >> (k + 1));
                };
                f32x4 Y, YT;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int sl = 4 * l4 + e;
                    const float id = sl == l15 ? 1.f : 0.f;
                    Y[e] = id - (joins(0, sl, l15) ? Mn[e] : 0.f);    // Y_1 = I - E_0
                    YT[e] = id - (joins(0, l15, sl) ? MT[e] : 0.f);
                }
#pragma unroll
                for (int k = 1; k < 4; ++k) {
                    f32x4 ET;   // acc(E_k^T)
#pragma unroll
                    for (int e = 0; e < 4; ++e) ET[e] = joins(k, l15, 4 * l4 + e) ? MT[e] : 0.f;
                    const f32x4 P = mfma16z(cvt4(ET), cvt4(Y));     // E_k Y_k
                    const f32x4 Yn = mfma16(cvt4(-YT), cvt4(P), Y); // Y_k - Y_k P
                    YT = mfma16(cvt4(-P), cvt4(YT), YT);            // Y_k^T - P^T Y_k^T
                    Y = Yn;
                }
                // acc(Y): Y[4 l4 + e][l15] -> T^T[s = l15][r] = Y[r][s] beta_s and
                // Y^T[b][c = l15][r]
                *reinterpret_cast<bf16x4 *>(&sm.TT[(16 * b + l15) * PCT + 16 * b + 4 * l4]) = cvt4(Y * bl);
                *reinterpret_cast<bf16x4 *>(&sm.YT[(16 * b + l15) * PY + 4 * l4]) = cvt4(Y);
                if (b >= 1) putL(b, b - 1, aoff);
            }
            if (hasS) {
                // outputs of chunk j-1, row block w.  O^T = U^T P^T + (Qt S0^T)^T:
                // lane holds columns 16 jv + 4 l4 .. +3 of output row 16 I + l15.
                const int I = w;
                const bf16x8 p0 = frag_cols(sm.PT, PCT, 0, 16 * I, lane);
                bf16x8 p1 = {};
                if (I >= 2) p1 = frag_cols(sm.PT, PCT, 32, 16 * I, lane);
                f32x4 ov[2];
#pragma unroll
                for (int jv = 0; jv < 2; ++jv) {
                    const f32x4 qs = *reinterpret_cast<const f32x4 *>(&sm.QS[((4 * jv + I) * 64 + lane) * 4]);
                    f32x4 o = mfma32(frag_rows(sm.UT, PC, 16 * jv, 0, lane), p0, qs);
                    if (I >= 2) o = mfma32(frag_rows(sm.UT, PC, 16 * jv, 32, lane), p1, o);
                    ov[jv] = o * a.scale;
                }
                const long long tc = t0 + (j - 1) * C;
                const int Cc = valid_rows(j - 1);
                const unsigned rowb = (unsigned)(tokstride * 2);
                const rsrc_t ro = make_rsrc(og + (size_t)tc * tokstride, a.o ? (Cc - 1) * rowb + BV * 2 : 0u);
#pragma unroll
                for (int jv = 0; jv < 2; ++jv)
                    bstore8s(ro, (16 * I + l15) * rowb + 2 * (16 * jv + 4 * l4), 0u, cvt4(ov[jv]));
            }
        } else {
            if (hasS) {
                // state update of chunk j-1 (key blocks of this wave)
                const int I = w - 4;
                bf16x8 uf[2][2];
#pragma unroll
                for (int jv = 0; jv < 2; ++jv) {
                    uf[jv][0] = frag_rows(sm.UT, PC, 16 * jv, 0, lane);
                    uf[jv][1] = frag_rows(sm.UT, PC, 16 * jv, 32, lane);
                }
                // S^T <- e^{b_C} (.) S^T + Kh^T U  (chunk j-1: parity 1 - PAR):
                // e^{b_C} (.) (S^T + Kb^T U), or for a wide chunk with
                // Kh_J = KE_J (.) e^{b_C - R_{J+1}} (the lane's channel is
                // 16 Jk + l15 and its tokens lie in blocks lane >> 5 (first
                // fragment) and 2 + (lane >> 5) (second))
#pragma unroll
                for (int kb = 0; kb < SBK; ++kb) {
                    const int Jk = SBK * I + kb;
                    const int jc = 16 * Jk + 4 * l4;
                    const f32x4 gm = *reinterpret_cast<const f32x4 *>(&sm.gam[1 - PAR][jc]);
                    bf16x8 k0f = frag_cols(sm.Kb[1 - PAR], PD, 0, 16 * Jk, lane);
                    bf16x8 k1f = frag_cols(sm.Kb[1 - PAR], PD, 32, 16 * Jk, lane);
                    if (REF) {
                        const int chn = 16 * Jk + l15;
                        const float f0 = sm.FU[1 - PAR][lane >> 5][chn];
                        const float f1 = (lane >> 5) ? 1.f : sm.FU[1 - PAR][2][chn];
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            k0f[u] = (bf16)((float)k0f[u] * f0);
                            k1f[u] = (bf16)((float)k1f[u] * f1);
                        }
                    }
#pragma unroll
                    for (int jv = 0; jv < 2; ++jv) {
                        f32x4 sv;
                        if (REF) {
                            sv = mfma32(k0f, uf[jv][0], St[kb][jv] * gm);
                            sv = mfma32(k1f, uf[jv][1], sv);
                        } else {
                            sv = mfma32(k0f, uf[jv][0], St[kb][jv]);
                            sv = mfma32(k1f, uf[jv][1], sv) * gm;
                        }
                        St[kb][jv] = sv;
                        *reinterpret_cast<bf16x4 *>(&sm.S[(16 * jv + l15) * PD + jc]) = cvt4(sv);
                        if (a.states && j < nch)   // the state entering chunk j
                            *reinterpret_cast<f32x4 *>(a.states + ((size_t)(cbase + j) * a.H + h) * D * D +
                                                       (size_t)(i0 + 16 * jv + l15) * D + jc) = sv;
                    }
                }
            }
            if (hasP && w < 7) {
                // blocks (2,0), (3,0), (3,1) of A and P
                const int I = w == 4 ? 2 : 3, J = w == 6 ? 1 : 0;
                // wide: against KE_J (.) e^{R_I - R_{J+1}} (at most 1)
                bf16x8 kf[KD], qf[KD], bf[KD];
                frags(sm.K, I, kf);
                frags(sm.Q, I, qf);
                frags(sm.Kb[PAR], J, bf);
                if (REF) {
#pragma unroll
                    for (int kk = 0; kk < KD; ++kk) scale_frag(bf[kk], kk, sm.FD[I == 2 ? 4 : (J == 0 ? 5 : 6)]);
                }
                f32x4 aoff;
                gram(kf, qf, bf, aoff, poff);
                putL(I, J, aoff);
            }
        }
        if (j + 2 < nch) scan(L, par_tag);
        load_g(L, j + 3);
        __syncthreads();

        // ================= phase C ========================================
        if (hasP) {
            if (w == 0) {
                // off-diagonal blocks of T:  Y_ij = -Y_ii sum_{k=j}^{i-1} L_ik Y_kj
                // on 16x16x16 MFMAs (A operand: row l15, cols 4*l4..+3;
                // B operand: rows 4*l4..+3, col l15 == the accumulator layout)
                auto opL = [&](int bi, int bk) -> bf16x4 {   // L_ik[l15][4*l4..] = L^T_ik[4*l4..][l15]
                    return frag_col4(sm.LTo[bi * (bi - 1) / 2 + bk], PY, 0, 0, lane);
                };
                auto opYA = [&](int bi) -> bf16x4 {   // Y_ii[l15][4*l4..] = Y^T[4*l4..][l15]
                    return frag_col4(sm.YT, PY, 16 * bi, 0, lane);
                };
                auto opYB = [&](int bj) -> bf16x4 {   // Y_jj[4*l4..][l15] = Y^T[l15][4*l4..]
                    return *reinterpret_cast<const bf16x4 *>(&sm.YT[(bj * 16 + l15) * PY + 4 * l4]);
                };
                const float bt0 = sm.beta[l15], bt1 = sm.beta[16 + l15], bt2 = sm.beta[32 + l15];
                const f32x4 z0 = {0.f, 0.f, 0.f, 0.f};
                const bf16x4 B00 = opYB(0), B11 = opYB(1), B22 = opYB(2);
                const bf16x4 A11 = opYA(1), A22 = opYA(2), A33 = opYA(3);
                const bf16x4 L10 = opL(1, 0), L21 = opL(2, 1), L32 = opL(3, 2);
                const bf16x4 L20 = opL(2, 0), L31 = opL(3, 1), L30 = opL(3, 0);
                const f32x4 Y10 = -mfma16(A11, cvt4(mfma16(L10, B00, z0)), z0);
                const f32x4 Y21 = -mfma16(A22, cvt4(mfma16(L21, B11, z0)), z0);
                const f32x4 Y32 = -mfma16(A33, cvt4(mfma16(L32, B22, z0)), z0);
                const f32x4 Y20 = -mfma16(A22, cvt4(mfma16(L21, cvt4(Y10), mfma16(L20, B00, z0))), z0);
                const f32x4 Y31 = -mfma16(A33, cvt4(mfma16(L32, cvt4(Y21), mfma16(L31, B11, z0))), z0);
                const f32x4 Y30 = -mfma16(
                    A33, cvt4(mfma16(L32, cvt4(Y20), mfma16(L31, cvt4(Y10), mfma16(L30, B00, z0)))), z0);
                // T_ij = Y_ij diag(beta_j) -> T^T[s][r..r+3]
                auto putT = [&](int bi, int bj, f32x4 yv, float bt) {
                    const int s = 16 * bj + l15;
                    *reinterpret_cast<bf16x4 *>(&sm.TT[s * PCT + 16 * bi + 4 * l4]) = cvt4(yv * bt);
                };
                putT(1, 0, Y10, bt0);
                putT(2, 1, Y21, bt1);
                putT(3, 2, Y32, bt2);
                putT(2, 0, Y20, bt0);
                putT(3, 1, Y31, bt1);
                putT(3, 0, Y30, bt0);
            } else if (w >= 4) {
                // Qt S0^T (for the outputs, transposed, to LDS) and
                // X = V - Kt S0^T, row block w-4: Kt = KR (.) e^{R_I},
                // Qt = QR (.) e^{R_I}
                const int I = w - 4;
                const int r0 = 16 * I + 4 * l4;
                bf16x8 kf[KD], qf[KD];
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) {
                    kf[kk] = frag_rows(sm.K, PD, 16 * I, 32 * kk, lane);
                    qf[kk] = frag_rows(sm.Q, PD, 16 * I, 32 * kk, lane);
                }
                if (REF && I > 0) {
#pragma unroll
                    for (int kk = 0; kk < KD; ++kk) {
                        scale_frag(kf[kk], kk, sm.FX[PAR][I - 1]);
                        scale_frag(qf[kk], kk, sm.FX[PAR][I - 1]);
                    }
                }
#pragma unroll
                for (int jv = 0; jv < 2; ++jv) {
                    bf16x8 sf[KD];
#pragma unroll
                    for (int kk = 0; kk < KD; ++kk) sf[kk] = frag_rows(sm.S, PD, 16 * jv, 32 * kk, lane);
                    f32x4 x = {0.f, 0.f, 0.f, 0.f}, o = x;
#pragma unroll
                    for (int kk = 0; kk < KD; ++kk) {
                        x = mfma32(kf[kk], sf[kk], x);
                        o = mfma32(sf[kk], qf[kk], o);
                    }
                    const int iv = 16 * jv + l15;
                    const bf16x4 vr4 = frag_col4(sm.V, PV, 16 * I, 16 * jv, lane);   // V[r0 + e][iv]
                    f32x4 xv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) xv[e] = (float)vr4[e] - x[e];
                    *reinterpret_cast<bf16x4 *>(&sm.XT[iv * PC + r0]) = cvt4(xv);
                    *reinterpret_cast<f32x4 *>(&sm.QS[((4 * jv + I) * 64 + lane) * 4]) = o;
                }
            }
            // P(j) blocks computed in phase B
            if (w < 4) {
                putP(w, w, pdiag);
                if (w >= 1) putP(w, w - 1, poff);
            } else if (w < 7) {
                putP(w == 4 ? 2 : 3, w == 6 ? 1 : 0, poff);
            }
        }
        if (j + 2 < nch) prefix(PAR);
        if (hasG) gate(L, std::integral_constant<int, 1 - PAR>{});
        load_qkvb(L, j + 2, PAR);
        __syncthreads();
    };

    // ---- prologue: chunks 0 and 1 scanned, chunk 0 gated, chunk 1 loaded
    {
        const LI L(tid0);
        // unconditional even without a chunk (the loads then return zeros):
        // every path waits on these registers before the loop
        load_g(L, 0);
        load_qkvb(L, 0, 0);
        if (RAW) softplus_g(L, 0);
        scan(L, std::integral_constant<int, 0>{});
        load_g(L, 1);
        __syncthreads();
        prefix(0);
        if (RAW) softplus_g(L, 1);
        scan(L, std::integral_constant<int, 1>{});
        load_g(L, 2);
        __syncthreads();
        prefix(1);
        gate(L, std::integral_constant<int, 0>{});
        load_qkvb(L, 1, 1);
    }

    // iterations j = 0..nch: iteration 0 has no state chunk and iteration nch
    // no prep chunk; the ones between have both and are specialised for it,
    // so each wave's work in a phase is straight-line code.  They run in
    // (odd, even) pairs, so the loop is always entered from the end of an even
    // iteration and the loads in flight at its head are always the same.
    if (nch > 0) {
        using E = std::integral_constant<int, 0>;
        using O = std::integral_constant<int, 1>;
        iteration(E{}, std::false_type{}, std::true_type{}, 0);
        // no loads in flight on entry (vmcnt(0), other counters left as
        // they are): the loop's waits then follow from its own body alone,
        // whatever registers the peeled iteration loaded
        __builtin_amdgcn_s_waitcnt(0x0F70);
        long long j = 1;
        for (; j + 1 < nch; j += 2) {
            iteration(O{}, std::true_type{}, std::true_type{}, j);
            iteration(E{}, std::true_type{}, std::true_type{}, j + 1);
        }
        if (j < nch) {
            iteration(O{}, std::true_type{}, std::true_type{}, j);
            ++j;
        }
        if (j & 1) iteration(O{}, std::true_type{}, std::false_type{}, j);
        else       iteration(E{}, std::true_type{}, std::false_type{}, j);
    }
    // The plain pass ran every chunk; if one of them was wide its results
    // are void, and the reference pass redoes the pair from its start (all
    // outputs, states and the final state)
    if (!REF) {
        const bool wide_hit = __builtin_amdgcn_readfirstlane(sm.wide_any) != 0;
        if (tile == 0 && tid0 == 0) a.unit_wide[(size_t)n * a.H + h] = wide_hit ? 1 : 0;
        if (wide_hit) return;
    }

    if (float *htp = seq_ht<D>(a, n, h)) {
        const LI L(tid0);
        if (L.w >= 4) {
#pragma unroll
            for (int kb = 0; kb < SBK; ++kb) {
#pragma unroll
                for (int jv = 0; jv < 2; ++jv) {
                    const int j = 16 * (SBK * (L.w - 4) + kb) + 4 * L.l4;
                    const int iv = 16 * jv + L.l15;
                    *reinterpret_cast<f32x4 *>(htp + (size_t)(i0 + iv) * D + j) = St[kb][jv];
                }
            }
        }
    }
}

// Longest sequence first: rank = number of sequences that are longer, or
// equally long with a smaller index (a stable descending order).
__global__ __launch_bounds__(256) void schedule_kernel(const int32_t *cu, int N, int32_t *order) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    const int len = cu[n + 1] - cu[n];
    int rank = 0;
    for (int m = 0; m < N; ++m) {
        const int lm = cu[m + 1] - cu[m];
        rank += (lm > len) || (lm == len && m < n);
    }
    order[rank] = n;
}

}  // namespace

hipError_t launch_prefill_chunked(int D, const PrefillArgs &a, hipStream_t s) {
    if (!a.channel_gate) return launch_prefill_chain(D, a, s);
    const long long units = (long long)a.N * a.H;
    if (units <= 0) return hipSuccess;
    const int ntile = D / BV;
    const long long blocks = ((units + 7) / 8) * 8 * ntile;
    dim3 grid((unsigned)blocks), block(NT);
    // the plain pass, then the reference pass over the pairs it marked
    if (!a.unit_wide) return hipErrorInvalidValue;
    if (a.xg) {
        if (D == 128) hipLaunchKernelGGL((chunked_kernel<128, true, false>), grid, block, 0, s, a);
        else          hipLaunchKernelGGL((chunked_kernel<64, true, false>), grid, block, 0, s, a);
    } else {
        if (D == 128) hipLaunchKernelGGL((chunked_kernel<128, false, false>), grid, block, 0, s, a);
        else          hipLaunchKernelGGL((chunked_kernel<64, false, false>), grid, block, 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.xg) {
        if (D == 128) hipLaunchKernelGGL((chunked_kernel<128, true, true>), grid, block, 0, s, a);
        else          hipLaunchKernelGGL((chunked_kernel<64, true, true>), grid, block, 0, s, a);
    } else {
        if (D == 128) hipLaunchKernelGGL((chunked_kernel<128, false, true>), grid, block, 0, s, a);
        else          hipLaunchKernelGGL((chunked_kernel<64, false, true>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_varlen_schedule(const int32_t *cu_seqlens, int N, int32_t *order,
                                  hipStream_t s) {
    if (N <= 0) return hipSuccess;
    dim3 grid((unsigned)((N + 255) / 256)), block(256);
    hipLaunchKernelGGL(schedule_kernel, grid, block, 0, s, cu_seqlens, N, order);
    return hipGetLastError();
}

}  // namespace gdr
