// chunked_chain.hip -- chunked prefill of the gated delta rule for the scalar
// gate (Gated DeltaNet) in two kernels: the chunk-local inverse of every
// chunk in parallel, then the recurrence over chunks with the state on
// dedicated waves.
//
// Chunked form ("Super Apriel: One Checkpoint, Many Speeds", gist.science
// summary 2a, for the recurrence; the reorganisation into chunks is derived
// in chunked.hip).  For a chunk of C = 64 tokens entering with state S (Dv x
// Dk), b_r the in-chunk cumulative log gate and beta_r the write strength:
//     A[r][s] = e^{b_r - b_s} k_r.k_s (s < r),  P[r][s] = e^{b_r - b_s} q_r.k_s
//     (s <= r),  L = diag(beta) A,  T = (I + L)^{-1} diag(beta)
//     X = V - diag(e^b) K S^T,   U = T X
//     O = scale (diag(e^b) Q S^T + P U)
//     S^T <- e^{b_C} S^T + K^T diag(e^{b_C - b}) U
//
// prep_kernel (one workgroup per chunk and head) forms what U needs that
// does not depend on the state, and writes it with the chunk's decay factors
// to a record in the workspace, laid out as MFMA A operands (one 8- or
// 16-byte piece per lane and operand): the diagonal 16x16 blocks of
// T = N diag(beta), N = (I + L)^{-1}, and the blocks A_IJ (I > J) of A
// negated.  The recurrence kernel then solves (I + L) U = diag(beta) X by
// block forward substitution,
//     U_I = T_II (X_I - sum_{J<I} A_IJ U_J),
// whose terms are bounded by |A| <= 1 and |U|, rather than applying the full
// T, whose entries can grow large and cancel when beta A nears 1 (keys close
// to one direction).  Each N_II is formed in fp32 by forward substitution,
// one column per lane, and rounded once; a finite series in the nilpotent
// part would add terms that grow like binomial coefficients there.
//
// chain_kernel (one workgroup per sequence, head and 32-wide slice of Dv)
// walks the chunks in order.  The only dependency from chunk to chunk is the
// state, through X, U and the update.  Two "chain" waves (SIMDs 0 and 1)
// each own 16 of the 32 value columns and keep their slice of S^T (Dk x 16,
// fp32) in accumulator registers for the whole sequence; they do nothing but
// X, U and the update, and publish S^T and U as bf16 MFMA operands.  Four
// output waves (SIMDs 2 and 3) each own a 16-row block and form P and O one
// chunk behind.  Two staging waves (SIMDs 0 and 1, no MFMA work) bring the
// k rows, the v slice and the chunk's record (T and the decay factors)
// of chunk c+2, and the q rows of chunk c+1, into LDS while chunk c runs,
// their global loads (whole 128-byte lines) issued two iterations before
// the LDS stores.
// One barrier per chunk; between barriers c-1 and c (iteration c):
//   chain:   X, U and the state update of chunk c from registers, with
//            the LDS operands of chunk c+1 read into registers while the
//            update's MFMAs run (each K^T block right after its last use),
//            then publish U (by chunk parity) and the new S^T (kept as the
//            next X's operand), and read the v slice and e^b of chunk c+1
//   output:  O of chunk c-1 (U of c-1 was published in iteration c-1), then
//            diag(e^b) Q S^T and P of chunk c (S^T entering c likewise)
//   staging: chunk c+2 (k, v, record) and the q rows of chunk c+1 from
//            registers into LDS, global loads of chunk c+4 and of the q rows
//            of chunk c+3
// Every LDS value is written in one iteration and read in the next (U, S^T
// and the q rows are double-buffered by chunk parity, the other staged data
// are held in three slots), so the one barrier orders every producer before
// its reader.
#include "gdr_internal.h"
#include "device_util.h"

namespace gdr {
namespace {

constexpr int C = 64;        // chunk length
constexpr int BV = 32;       // value columns per recurrence workgroup

__device__ inline int tri(int i, int j) { return i * (i + 1) / 2 + j; }   // block (i >= j)
__device__ inline int ltri(int i, int j) { return i * (i - 1) / 2 + j; }  // block (i > j)

// ===========================================================================
// prep_kernel: T of one (chunk, head)
// ===========================================================================
// 27,136 bytes for the scalar gate, so that six workgroups fit a CU's LDS
template <int D, bool RAW> struct PrepSmem {
    static constexpr int PD = D + 8;    // rows padded by 16 bytes
    union alignas(16) {
        bf16 K[C * PD];                 // k rows, read by the Gram blocks
        float Nd[4][256];               // then N_bb, [r][s]
    };
    alignas(16) float MT[4][256];       // L_bb^T, [s][r] (strictly lower L_bb)
    // the record's operands as tiles (lane l: row l & 15, columns 4 (l >> 4)
    // .. +3): T_00, T_11, T_22, T_33, -A_10, -A_32, -A_20, -A_21, -A_30, -A_31
    alignas(16) bf16 TT[10 * 256];
    alignas(16) float fb[C];            // b_r
    alignas(16) float fbeta[C];         // beta_r
    alignas(16) float frk[RAW ? C : 1]; // 1 / |k_r| (fused preprocessing)
};

// RAW (fused preprocessing): gate and beta from their logits, the Gram
// blocks scaled by the inverse key norms 1/|k_r| 1/|k_s|, and a 6 KiB
// record whose rows are b_r log2(e), e^{b_C - b_r}/|k_r|, e^{b_r}/|k_r|
// and 1/|k_r| (the chain kernel applies 1/|q_r| itself).
// Every gate log is raised to kGateFloor first, so that the prefix sums and
// their differences stay finite for any gate a in [0, 1].
template <int D, bool RAW>
__global__ __launch_bounds__(256) void prep_kernel(PrefillArgs a) {
    using Sm = PrepSmem<D, RAW>;
    constexpr int PD = Sm::PD;
    constexpr int KD = D / 32;
    constexpr int CG = D / 8;           // 16-byte pieces per row
    constexpr int NPC = C * CG / 256;
    static_assert(NPC >= 1 && (C * CG) % 256 == 0, "staging layout");
    static_assert(kTileBytes == 5 * 1024 + 3 * C * 4, "tile record: T operands, three factor rows");
    constexpr size_t REC = RAW ? kTileBytesRaw : kTileBytes;
    __shared__ Sm sm;

    // ---- which chunk: ci counts chunks over all sequences.  Workgroups are
    //      handed to the eight XCDs in turn; each XCD takes a contiguous run
    //      of (chunk, head) units, so the heads of one chunk share an XCD and
    //      the lines of g and beta they read ([token, head] rows) are
    //      fetched into one L2 only
    const long long units = a.max_chunks * a.H;
    const long long per_xcd = (units + 7) / 8;
    const long long unit = (long long)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (unit >= units) return;
    const int h = (int)(unit % a.H);
    const long long ci = unit / a.H;
    long long t0, t1, c;
    if (a.cu_seqlens) {
        if (ci >= a.chunk_base[a.N]) return;
        int lo = 0, hi = a.N - 1;   // the last sequence whose first chunk is <= ci
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.chunk_base[mid] <= ci) lo = mid;
            else hi = mid - 1;
        }
        t0 = a.cu_seqlens[lo];
        t1 = a.cu_seqlens[lo + 1];
        c = ci - a.chunk_base[lo];
    } else {
        const long long nch = (a.T + C - 1) / C;
        const long long n = ci / nch;
        c = ci - n * nch;
        t0 = n * a.T;
        t1 = t0 + a.T;
    }
    const long long tc = t0 + c * C;
    const int Cc = (int)(t1 - tc < C ? t1 - tc : C);
    const size_t tokstride = (size_t)a.H * D;
    const unsigned rowb = (unsigned)(tokstride * 2);
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l15 = lane & 15, q4 = lane >> 4;

    // ---- k rows (rows past the sequence read as zeros), gate sums
    {
        const size_t base = (size_t)tc * tokstride + (size_t)h * D;
        const rsrc_t rks = make_rsrc(static_cast<const bf16 *>(a.k) + base,
                                     (unsigned)(Cc - 1) * rowb + D * 2);
        bf16x8 vk[NPC];
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int p = i * 256 + tid;
            vk[i] = bload16(rks, (p / CG) * rowb + 16 * (p % CG));
        }
        float gv = 0.f, bv = 0.f;
        if (w == 0) {
            const size_t gb = (size_t)tc * a.H + h;
            if (RAW) {
                // rows past the sequence end keep g = 0 and beta = 0
                const unsigned hx = (unsigned)(a.H * 2);
                const unsigned xext = (unsigned)(Cc - 1) * hx + 2;
                const float xg = bf16_bits_to_float(
                    bload2(make_rsrc(static_cast<const bf16 *>(a.xg) + gb, xext), lane * hx));
                const float xb = bf16_bits_to_float(
                    bload2(make_rsrc(static_cast<const bf16 *>(a.xb) + gb, xext), lane * hx));
                gv = lane < Cc ? neg_softplus(xg, a.gate_scale) : 0.f;
                bv = lane < Cc ? logistic(xb) : 0.f;
            } else {
                const unsigned hb = (unsigned)(a.H * 4);
                const unsigned gext = (unsigned)(Cc - 1) * hb + 4;
                gv = bload4(make_rsrc(a.g + gb, gext), lane * hb);
                bv = bload4(make_rsrc(a.beta + gb, gext), lane * hb);
            }
            gv = __builtin_fmaxf(gv, kGateFloor);
        }
        if (RAW) {
            // |k_r|^2 over the CG consecutive lanes that hold row r
#pragma unroll
            for (int i = 0; i < NPC; ++i) {
                float ss = 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u) ss = __builtin_fmaf((float)vk[i][u], (float)vk[i][u], ss);
                ss = sum_group<CG>(ss);
                const int p = i * 256 + tid;
                if (p % CG == 0) sm.frk[p / CG] = inv_norm(ss);
            }
        }
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int p = i * 256 + tid;
            *reinterpret_cast<bf16x8 *>(&sm.K[(p / CG) * PD + 8 * (p % CG)]) = vk[i];
        }
        if (w == 0) {
            sm.fb[lane] = wave_prefix_sum(gv);
            sm.fbeta[lane] = bv;
        }
    }
    __syncthreads();

    auto frags = [&](int blk, bf16x8 (&f)[KD]) {
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) f[kk] = frag_rows(sm.K, PD, 16 * blk, 32 * kk, lane);
    };
    // G = K_J K_I^T: lane holds s = 16J + 4 q4 + e, r = 16I + l15
    auto gram = [&](const bf16x8 (&kj)[KD], const bf16x8 (&ki)[KD]) -> f32x4 {
        f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) g = mfma32(kj[kk], ki[kk], g);
        return g;
    };
    // Gram block (I, J) of the normalised keys: times 1/|k_r| 1/|k_s|
    auto knorm = [&](int I, int J, f32x4 g) -> f32x4 {
        if (!RAW) return g;
        const float nr = sm.frk[16 * I + l15];
        const f32x4 ns = *reinterpret_cast<const f32x4 *>(&sm.frk[16 * J + 4 * q4]);
        return g * ns * nr;
    };
    // block (I, J) of the chunk: I == J: L_II = strict_lower(diag(beta) A_II)
    // in fp32, transposed, for the substitution; I > J: -A_IJ as a tile.
    // A[r][s] = e^{b_r - b_s} k_r.k_s (s < r, so the factor is at most 1)
    auto put_A = [&](int I, int J, int tile, f32x4 g) {
        const float br = sm.fb[16 * I + l15];
        const f32x4 bs = *reinterpret_cast<const f32x4 *>(&sm.fb[16 * J + 4 * q4]);
        g = knorm(I, J, g);
        f32x4 av;
#pragma unroll
        for (int e = 0; e < 4; ++e) av[e] = ex(br - bs[e]) * g[e];
        if (I == J) {
            const float betar = sm.fbeta[16 * I + l15];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int sl = 4 * q4 + e;
                sm.MT[I][16 * sl + l15] = sl < l15 ? betar * av[e] : 0.f;
            }
        } else {
            tile_st(sm.TT + tile * 256, lane, -av);
        }
    };

    // ---- wave w: blocks (w, w) and, below the diagonal, w0: (1,0), (3,0)
    //      w1: (2,1), (3,1)  w2: (2,0)  w3: (3,2)
    {
        const int b = w;
        bf16x8 kd[KD];
        frags(b, kd);
        put_A(b, b, 0, gram(kd, kd));
        // tiles: (1,0) 4, (3,2) 5, (2,0) 6, (2,1) 7, (3,0) 8, (3,1) 9
        const int J = b < 2 ? b : (b == 2 ? 0 : 2);
        const int I0 = b < 2 ? b + 1 : (b == 2 ? 2 : 3);
        const int t0 = b == 0 ? 4 : (b == 1 ? 7 : (b == 2 ? 6 : 5));
        bf16x8 kj[KD], ki[KD];
        frags(J, kj);
        frags(I0, ki);
        put_A(I0, J, t0, gram(kj, ki));
        if (b < 2) {
            frags(3, ki);
            put_A(3, J, b == 0 ? 8 : 9, gram(kj, ki));
        }
    }
    __syncthreads();

    // ---- N_bb = (I + L_bb)^{-1} in fp32 by forward substitution, lane
    //      16 b + c of wave 0 taking column c of block b: once entry m of the
    //      column is final, column m of L_bb updates the entries below it
    if (w == 0) {
        const int b = lane >> 4, c = lane & 15;
        const float *Lt = sm.MT[b];
        float n[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) n[r] = r == c ? 1.f : 0.f;
        auto lcol = [&](int m, f32x4 (&R)[4]) {   // column m: four reads, one address per block
#pragma unroll
            for (int v = 0; v < 4; ++v) R[v] = *reinterpret_cast<const f32x4 *>(&Lt[16 * m + 4 * v]);
        };
        f32x4 Lc[4], Ln[4];
        lcol(0, Lc);
#pragma unroll
        for (int m = 0; m < 15; ++m) {
            if (m + 1 < 15) lcol(m + 1, Ln);
#pragma unroll
            for (int r = m + 1; r < 16; ++r) n[r] -= Lc[r >> 2][r & 3] * n[m];
#pragma unroll
            for (int v = 0; v < 4; ++v) Lc[v] = Ln[v];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.Nd[b][16 * r + c] = n[r];
    }
    __syncthreads();
    // ---- T_bb = N_bb diag(beta_b) as tiles, rounded to bf16 once
    {
        const int b = w;
        const f32x4 nv = *reinterpret_cast<const f32x4 *>(&sm.Nd[b][16 * l15 + 4 * q4]);
        const f32x4 bv = *reinterpret_cast<const f32x4 *>(&sm.fbeta[16 * b + 4 * q4]);
        tile_st(sm.TT + b * 256, lane, nv * bv);
    }
    __syncthreads();

    // ---- the chunk's record in the workspace: the pairs (-A_20 | -A_21) and
    //      (-A_30 | -A_31), a 16-byte piece per lane (the A operands of a
    //      16x16x32 MFMA over the tokens of blocks 0 and 1), then T_00 ..
    //      T_33, -A_10 and -A_32, 8 bytes per lane (16x16x16 MFMA A
    //      operands).  Then two rows of 64 fp32 values from b_r, the in-chunk
    //      inclusive prefix sums of the gate logs: b_r log2(e) itself (the
    //      recurrence forms e^{b_r} and e^{b_r - b_s}, s <= r, from it, so
    //      no factor ever exceeds 1) and e^{b_C - b_r}.
    {
        const size_t rec = (size_t)(ci * a.H + h) * REC;
        char *dst = static_cast<char *>(a.tiles) + rec;
        if (tid < 2 * 64) {
            const int pr = tid >> 6, l = tid & 63;
            reinterpret_cast<bf16x8 *>(dst)[tid] = cat8(tile_ld(sm.TT + (6 + 2 * pr) * 256, l),
                                                        tile_ld(sm.TT + (7 + 2 * pr) * 256, l));
        }
        for (int i = tid; i < 6 * 64; i += 256)
            reinterpret_cast<bf16x4 *>(dst + 2048)[i] = tile_ld(sm.TT + (i >> 6) * 256, i & 63);
        if (tid >= 128 && tid < 128 + C) {
            const int r = tid - 128;
            float *f = reinterpret_cast<float *>(dst + 5120);
            const float b = sm.fb[r];
            f[r] = b * kLog2e;
            if (RAW) {
                const float nk = sm.frk[r];
                f[C + r] = ex(sm.fb[C - 1] - b) * nk;
                f[2 * C + r] = ex(b) * nk;
                f[3 * C + r] = nk;
            } else {
                f[C + r] = ex(sm.fb[C - 1] - b);
                f[2 * C + r] = ex(b);
            }
        }
    }
}

// ===========================================================================
// chain_kernel: the recurrence over chunks
// ===========================================================================
// the chunk's workspace record as the prep kernel writes it
template <bool RAW> struct TRecT {
    bf16x8 pairs[2][64];            // (-A_20 | -A_21), (-A_30 | -A_31)
    bf16x4 halves[6][64];           // T_00, T_11, T_22, T_33, -A_10, -A_32
    float lb[C];                    // b_r log2(e)
    float hs[C];                    // e^{b_C - b_r}
    float ek[C];                    // e^{b_r}
};
template <> struct TRecT<true> {
    bf16x8 pairs[2][64];
    bf16x4 halves[6][64];
    float lb[C];                    // b_r log2(e)
    float hs[C];                    // e^{b_C - b_r} / |k_r|
    float ek[C];                    // e^{b_r} / |k_r|
    float rk[C];                    // 1 / |k_r|
};

template <int D, bool RAW> struct ChainSmem {
    // k rows; a row stride of 8 x odd dwords keeps the 16-byte row fragment
    // reads free of bank conflicts (and halves those of the transpose reads,
    // against 4 x odd)
    static constexpr int PD = D + 16;
    static constexpr int KD = D / 32;
    // v slice rows [r][i]; a stride of 24 dwords puts the 8 rows that one
    // transpose load touches per half-wave on disjoint banks
    static constexpr int PV = BV + 16;
    using TRec = TRecT<RAW>;
    alignas(16) bf16 K[3][C * PD];      // by chunk mod 3
    alignas(16) bf16 Q[2][C * PD];      // by chunk parity
    alignas(16) bf16 V[3][C * PV];      // by chunk mod 3
    alignas(16) TRec TR[3];             // by chunk mod 3
    alignas(16) bf16x8 SB[2][2][KD][64];// S^T entering a chunk (by parity), per chain wave
    alignas(16) bf16x8 UB[2][2][2][64]; // U as operands (by parity), per chain wave
};

template <int D, bool RAW>
__global__ __launch_bounds__(512, 1) void chain_kernel(PrefillArgs a) {
    using Sm = ChainSmem<D, RAW>;
    constexpr size_t REC = RAW ? kTileBytesRaw : kTileBytes;
    constexpr int PD = Sm::PD;
    constexpr int PV = Sm::PV;
    constexpr int NTILE = D / BV;
    constexpr int KD = Sm::KD;          // 32-wide k steps over Dk
    constexpr int KS = D / 16;          // 16-row blocks of S^T
    constexpr int CG = D / 8;           // 16-byte pieces per k row
    // staged pieces (16 bytes) per chunk: k rows, v slice rows, T record
    constexpr int NKP = C * CG, NVP = C * BV / 8, NTP = (int)(REC / 16);
    constexpr int NST = NKP + NVP + NTP;
    constexpr int NI = (NST + 127) / 128;   // per staging thread
    static_assert(NKP % 64 == 0 && NVP % 64 == 0, "staging layout");
    static_assert(sizeof(typename Sm::TRec) == REC, "tile record layout");
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
    long long t0, t1, cbase;
    if (a.cu_seqlens) {
        t0 = a.cu_seqlens[n];
        t1 = a.cu_seqlens[n + 1];
        cbase = a.chunk_base[n];
    } else {
        t0 = (long long)n * a.T;
        t1 = t0 + a.T;
        cbase = (long long)n * ((a.T + C - 1) / C);
    }
    const int i0 = tile * BV;
    const size_t tokstride = (size_t)a.H * D;
    const unsigned rowb = (unsigned)(tokstride * 2);   // bytes between tokens
    const bf16 *qg = static_cast<const bf16 *>(a.q) + (size_t)h * D;
    const bf16 *kg = static_cast<const bf16 *>(a.k) + (size_t)h * D;
    const bf16 *vg = static_cast<const bf16 *>(a.v) + (size_t)h * D + i0;
    bf16 *og = static_cast<bf16 *>(a.o) + (size_t)h * D + i0;
    const long long nch = (t1 - t0 + C - 1) / C;
    // The output and staging waves run their loops in pairs of iterations
    // (two register sets) with one exit test per pair, so that the compiler
    // sees a single back edge and waits on each register set by the loads
    // issued after it (an exit test between the two halves gives it a path
    // on which the newest loads would be waited for at once).  All roles
    // pass nhalf + 1 barriers: iterations 0 .. nch do work, the rest (at most
    // one) find nothing to load or store.
    const long long nhalf = (nch + 2) & ~1LL;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l15 = lane & 15, q4 = lane >> 4;

    // rows of chunk c that exist (0 past the end and for c < 0); buffer
    // extents cover just these, so loads of other rows return zeros and
    // stores to them are dropped
    auto valid_rows = [&](long long c) -> int {
        const long long rem = t1 - (t0 + c * C);
        return (c < 0 || rem <= 0) ? 0 : (rem < C ? (int)rem : C);
    };
    // first token of chunk c (the sequence start for c < 0, whose extent is 0)
    auto chunk_tok = [&](long long c) -> long long { return c < 0 ? t0 : t0 + c * C; };
    auto extent = [&](long long c, unsigned row_bytes) -> unsigned {
        const int Cc = valid_rows(c);
        return Cc ? (unsigned)(Cc - 1) * rowb + row_bytes : 0u;
    };
    // The k index of the state.  A 16x16x32 MFMA sums over k; lane l of a
    // row-fragment operand (16 bytes of one k row) supplies k = 32 kk + 8 (l >> 4)
    // + u, u = 0..7.  The S^T accumulator blocks are numbered so that the pair
    // (2 kk, 2 kk + 1) supplies exactly these k as the other operand: block jk
    // holds rows 32 (jk >> 1) + 8 q4 + 4 (jk & 1) + e of S^T in lane (q4, e).
    auto srow = [&](int jk, int e) -> int { return 32 * (jk >> 1) + 8 * q4 + 4 * (jk & 1) + e; };
    const std::integral_constant<int, 0> R0;
    const std::integral_constant<int, 1> R1;
    // Value column (within the slice) of local column m of chain wave ib:
    // the two waves take alternate groups of four, so that an output lane's
    // four columns from each wave are eight adjacent ones (one 16-byte store)
    auto vcol = [](int ib, int m) -> int { return 8 * (m >> 2) + 4 * ib + (m & 3); };

    if (w < 2) {
        // =================================================================
        // chain waves: value columns vcol(ib, 0..15) of the slice
        // =================================================================
        const int ib = w;
        // S^T[srow(jk, e)][vcol(ib, l15)] (fp32); the four rows e of a block
        // are adjacent columns of S, so they move as one 16-byte access
        f32x4 St[KS];
        const size_t srow0 = (size_t)(i0 + vcol(ib, l15)) * D;
        const float *h0p = seq_h0<D>(a, n, h);
#pragma unroll
        for (int jk = 0; jk < KS; ++jk)
            St[jk] = h0p ? *reinterpret_cast<const f32x4 *>(h0p + srow0 + srow(jk, 0))
                         : f32x4{0.f, 0.f, 0.f, 0.f};
        // S^T entering the next chunk as bf16 operands: kept for its X and
        // published for the output waves (by chunk parity spar)
        bf16x8 Bs[KD];
        auto publish_state = [&](int spar) {
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) {
                Bs[kk] = acc_pair(St[2 * kk], St[2 * kk + 1]);
                sm.SB[spar][ib][kk][lane] = Bs[kk];
            }
        };
        // operands of a chunk, read an iteration ahead of their use: k row
        // fragments, K^T, the v slice, T and the decay factors (e^b from the
        // record, e^{b_C} formed from b_C)
        bf16x8 Kf[4][KD], KT[KS][2], Ap[2];
        bf16x4 Td[4], A10, A32;
        bf16x4 vv[4];
        f32x4 eb[4], hs[4];
        float gC = 0.f;
        // operands of the chunk in slot m3 read while the previous chunk's
        // state update runs: k row fragments, e^{b_C - b}, the diagonal
        // blocks of T and the blocks of -A below them
        auto prefetch_rows = [&](int m3) {
            const bf16 *Kc = sm.K[m3];
            const typename Sm::TRec &R = sm.TR[m3];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) Kf[rb][kk] = frag_rows(Kc, PD, 16 * rb, 32 * kk, lane);
                hs[rb] = *reinterpret_cast<const f32x4 *>(&R.hs[16 * rb + 4 * q4]);
                Td[rb] = R.halves[rb][lane];
            }
            A10 = R.halves[4][lane];
            A32 = R.halves[5][lane];
            Ap[0] = R.pairs[0][lane];
            Ap[1] = R.pairs[1][lane];
        };
        // the v slice, e^b (RAW: e^b / |k|) and e^{b_C} of the chunk in slot m3
        auto prefetch_veb = [&](int m3) {
            const bf16 *Vc = sm.V[m3];
            const typename Sm::TRec &R = sm.TR[m3];
            const float lbC = R.lb[C - 1];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                // rows 16 rb + 4 q4 .. +3 of column vcol(ib, l15), by one
                // transpose load: lane j of each 16-lane group addresses row
                // j >> 2 and the four columns vcol(ib, 4 (j & 3)) .. +3
                const bf16 *pv = Vc + (16 * rb + 4 * q4 + (l15 >> 2)) * PV + 8 * (l15 & 3) + 4 * ib;
                vv[rb] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)pv));
                eb[rb] = *reinterpret_cast<const f32x4 *>(&R.ek[16 * rb + 4 * q4]);
            }
            gC = __builtin_amdgcn_exp2f(lbC);
        };
        // K^T row block jk of the chunk in slot m3, by transpose loads: lane
        // j of each 16-lane group addresses k columns 32 (jk >> 1) + 8 (j & 3)
        // + 4 (jk & 1) .. +3, so output lane i receives k = srow(jk, .) for
        // row i of the block
        auto kt_load = [&](int m3, int jk) {
            const bf16 *Kc = sm.K[m3];
            const int pc = 32 * (jk >> 1) + 8 * (l15 & 3) + 4 * (jk & 1);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16 *p = Kc + (32 * kk + 4 * q4 + (l15 >> 2)) * PD + pc;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 16 * PD));
                KT[jk][kk] = cat8(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi));
            }
        };
        auto prefetch_kt = [&](int m3) {
            prefetch_veb(m3);
#pragma unroll
            for (int jk = 0; jk < KS; ++jk) kt_load(m3, jk);
        };
        publish_state(0);
        __syncthreads();                      // chunks 0 and 1 staged
        prefetch_rows(0);
        prefetch_kt(0);
        int m3 = 0;                           // c mod 3
        bool wide = false;                    // a chunk decays by more than e^80
        for (long long c = 0; c < nch; ++c) {
            const int par = (int)(c & 1);
            const int n3 = m3 == 2 ? 0 : m3 + 1;
            if (a.states) {                   // the state entering chunk c
                float *sp = a.states + ((size_t)(cbase + c) * a.H + h) * D * D + srow0;
#pragma unroll
                for (int jk = 0; jk < KS; ++jk) *reinterpret_cast<f32x4 *>(sp + srow(jk, 0)) = St[jk];
            }
            const float gCc = gC;             // e^{b_C} of chunk c
            wide |= !(gCc >= 1.8e-35f);       // e^{b_C} < e^-80
            // ---- X = V - diag(e^b) K S^T, U = T X and the state
            //      update, all from registers
            f32x4 X[4];
            {
                f32x4 xk[4];
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    xk[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KD; ++kk) xk[rb] = mfma32(Kf[rb][kk], Bs[kk], xk[rb]);
                }
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) X[rb][e] = (float)vv[rb][e] - eb[rb][e] * xk[rb][e];
            }
            // (I + L) U = diag(beta) X by block forward substitution,
            // U_I = T_II (X_I - sum_{J<I} A_IJ U_J), then
            // S^T <- e^{b_C} S^T + K^T diag(e^{b_C - b}) U
            bf16x8 Ub[2];
            {
                f32x4 U[4];
                U[0] = mfma16z(Td[0], cvt4(X[0]));
                U[1] = mfma16z(Td[1], cvt4(mfma16(A10, cvt4(U[0]), X[1])));
                const bf16x8 U01 = acc_pair(U[0], U[1]);
                U[2] = mfma16z(Td[2], cvt4(mfma32(Ap[0], U01, X[2])));
                U[3] = mfma16z(Td[3], cvt4(mfma16(A32, cvt4(U[2]), mfma32(Ap[1], U01, X[3]))));
                Ub[0] = acc_pair(U[0], U[1]);
                Ub[1] = acc_pair(U[2], U[3]);
                f32x4 Uh[4];
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) Uh[sb] = U[sb] * hs[sb];
                const bf16x8 Bh[2] = {acc_pair(Uh[0], Uh[1]), acc_pair(Uh[2], Uh[3])};
                // the next chunk's operands but K^T, in flight during the update
                __builtin_amdgcn_sched_barrier(0);
                prefetch_rows(n3);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int jk = 0; jk < KS; ++jk) {
                    f32x4 sv = St[jk] * gCc;
                    sv = mfma32(KT[jk][0], Bh[0], sv);
                    sv = mfma32(KT[jk][1], Bh[1], sv);
                    St[jk] = sv;
                    kt_load(n3, jk);   // the next chunk's K^T block, in flight during the rest
                }
            }
            // publish U and S^T; the rest of the next chunk's operands
            sm.UB[par][ib][0][lane] = Ub[0];
            sm.UB[par][ib][1][lane] = Ub[1];
            publish_state(par ^ 1);
            prefetch_veb(n3);
            __syncthreads();
            m3 = n3;
        }
        for (long long c = nch; c < nhalf; ++c) __syncthreads();   // outputs of the last chunk
        if (a.unit_wide && tile == 0 && w == 0 && lane == 0)
            a.unit_wide[(size_t)n * a.H + h] = wide ? 1 : 0;
        if (float *htp = seq_ht<D>(a, n, h)) {
#pragma unroll
            for (int jk = 0; jk < KS; ++jk) *reinterpret_cast<f32x4 *>(htp + srow0 + srow(jk, 0)) = St[jk];
        }
        return;
    }

    if (w >= 4 && w < 6) {
        // =================================================================
        // staging waves: k rows, the v slice and the record (T, factors) of
        // chunk c+2 into LDS in iteration c, from registers loaded in
        // iteration c-2 (two register sets)
        // =================================================================
        const int tl = tid - 256;
        bf16x8 rs[2][NI];
        constexpr int NQ = NKP / 128;         // q pieces per staging thread
        bf16x8 qs[2][NQ];
        auto q_load = [&](long long c, auto S) {
            constexpr int r = decltype(S)::value;
            const rsrc_t rq = make_rsrc(qg + (size_t)chunk_tok(c) * tokstride, extent(c, D * 2));
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int p = i * 128 + tl;
                qs[r][i] = bload16(rq, (p / CG) * rowb + 16 * (p % CG));
            }
        };
        auto q_store = [&](int slot, auto S) {
            constexpr int r = decltype(S)::value;
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int p = i * 128 + tl;
                *reinterpret_cast<bf16x8 *>(&sm.Q[slot][(p / CG) * PD + 8 * (p % CG)]) = qs[r][i];
            }
        };
        auto st_load = [&](long long c, auto S) {
            constexpr int r = decltype(S)::value;
            const size_t base = (size_t)chunk_tok(c) * tokstride;
            const rsrc_t rks = make_rsrc(kg + base, extent(c, D * 2));
            const rsrc_t rvs = make_rsrc(vg + base, extent(c, BV * 2));
            const bool have = valid_rows(c) > 0 && cbase + c < a.max_chunks;
            const size_t rec = (size_t)((have ? cbase + c : 0) * a.H + h) * REC;
            const rsrc_t rts = make_rsrc(static_cast<const char *>(a.tiles) + rec,
                                         have ? (unsigned)REC : 0u);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int p0 = i * 128 + 64 * (w - 4);   // this wave's first piece
                const int p = i * 128 + tl;
                if (p0 < NKP) {
                    rs[r][i] = bload16(rks, (p / CG) * rowb + 16 * (p % CG));
                } else if (p0 < NKP + NVP) {
                    const int pv = p - NKP;
                    rs[r][i] = bload16(rvs, (pv >> 2) * rowb + 16 * (pv & 3));
                } else {
                    rs[r][i] = bload16(rts, 16 * (p - NKP - NVP));
                }
            }
        };
        auto st_store = [&](int m3, auto S) {   // chunk c into slot m3 = c mod 3
            constexpr int r = decltype(S)::value;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int p0 = i * 128 + 64 * (w - 4);
                const int p = i * 128 + tl;
                if (p0 < NKP) {
                    *reinterpret_cast<bf16x8 *>(&sm.K[m3][(p / CG) * PD + 8 * (p % CG)]) = rs[r][i];
                } else if (p0 < NKP + NVP) {
                    const int pv = p - NKP;
                    *reinterpret_cast<bf16x8 *>(&sm.V[m3][(pv >> 2) * PV + 8 * (pv & 3)]) = rs[r][i];
                } else if (p < NST) {
                    reinterpret_cast<bf16x8 *>(&sm.TR[m3])[p - NKP - NVP] = rs[r][i];
                }
            }
        };
        // q rows go one chunk behind the rest: chunk c+1 into q slot
        // (c+1) mod 2 in iteration c, from registers loaded in iteration c-2
        st_load(0, R0);
        q_load(0, R0);
        st_store(0, R0);
        q_store(0, R0);
        st_load(1, R0);
        st_store(1, R0);
        // loads strictly in this order: the loop waits for each register set
        // by the number of loads issued after it, which assumes it
        st_load(2, R0);
        q_load(1, R1);
        q_load(2, R0);
        __builtin_amdgcn_sched_barrier(0);
        st_load(3, R1);
        __syncthreads();
        int m3 = 2;                           // (c + 2) mod 3
        for (long long c = 0; c < nhalf; c += 2) {
            st_store(m3, R0);
            q_store(1, R1);                   // chunk c + 1
            m3 = m3 == 2 ? 0 : m3 + 1;
            st_load(c + 4, R0);
            q_load(c + 3, R1);
            __syncthreads();
            st_store(m3, R1);
            q_store(0, R0);                   // chunk c + 2
            m3 = m3 == 2 ? 0 : m3 + 1;
            st_load(c + 5, R1);
            q_load(c + 4, R0);
            __syncthreads();
        }
        return;
    }

    // =====================================================================
    // output waves: row block RB of the chunk (waves 2, 3, 7, 6 take 0, 1, 2,
    // 3, so each of SIMDs 2 and 3 carries 1 + 4 or 2 + 3 blocks of P), both
    // value blocks (the columns of the two chain waves).  O^T = scale (S Q^T
    // diag(e^b) + U^T P^T) so that a lane ends up with four columns of one
    // output row per block, eight adjacent ones in all (vcol): the published
    // S^T and U serve as A operands, the q rows and P^T as B operands.  P^T
    // is formed in accumulator registers, so it feeds the MFMA directly.
    // Iteration c: O of chunk c-1 (U of chunk c-1 was published in iteration
    // c-1), then QS and P of chunk c (S^T entering chunk c was published in
    // iteration c-1, chunk c's k rows stay in their LDS slot until iteration
    // c+1 refills it, and its q rows were staged in iteration c-1).
    // =====================================================================
    auto out_loop = [&](auto RBc) {
        constexpr int RB = decltype(RBc)::value;
        constexpr int NP2 = (RB + 2) / 2;   // pairs of 16-token blocks J <= RB
        bf16x8 Pp[NP2];                     // P^T of the previous chunk, as B operand pairs
        f32x4 QSp[2];                       // (Q S^T)^T[vcol(ob, 4 q4 + e)][16 RB + l15], scaled by e^b
        // O of chunk c-1
        auto o_step = [&](long long c) {
            bf16x8 Au[2][NP2];
            const int up = (int)((c - 1) & 1);
#pragma unroll
            for (int ob = 0; ob < 2; ++ob)
#pragma unroll
                for (int k2 = 0; k2 < NP2; ++k2) Au[ob][k2] = sm.UB[up][ob][k2][lane];
            __builtin_amdgcn_sched_barrier(0);
            const rsrc_t ro = make_rsrc(og + (size_t)chunk_tok(c - 1) * tokstride, a.o ? extent(c - 1, BV * 2) : 0u);
            // lane (q4, l15): columns vcol(ob, 4 q4 + e) = 8 q4 + 4 ob + e of
            // row 16 RB + l15, eight adjacent columns over the two blocks
            f32x4 o[2];
#pragma unroll
            for (int ob = 0; ob < 2; ++ob) {
                o[ob] = QSp[ob];
#pragma unroll
                for (int k2 = 0; k2 < NP2; ++k2) o[ob] = mfma32(Au[ob][k2], Pp[k2], o[ob]);
            }
            bstore16s(ro, l15 * rowb + 16 * q4, 16 * RB * rowb,
                      cat8(cvt4(o[0] * a.scale), cvt4(o[1] * a.scale)));
        };
        // QS and P of chunk c (m3 = c mod 3)
        auto qp_step = [&](long long c, int m3) {
            const bf16 *Kc = sm.K[m3];
            const bf16 *Qc = sm.Q[(int)(c & 1)];
            bf16x8 As[2][KD], Kj[RB + 1][KD], Qr[KD];   // Qr: q rows 16 RB + l15
            f32x4 lbJ[RB + 1], rkJ[RB + 1];
#pragma unroll
            for (int ob = 0; ob < 2; ++ob)
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) As[ob][kk] = sm.SB[(int)(c & 1)][ob][kk][lane];
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) Qr[kk] = frag_rows(Qc, PD, 16 * RB, 32 * kk, lane);
#pragma unroll
            for (int J = 0; J <= RB; ++J) {
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) Kj[J][kk] = frag_rows(Kc, PD, 16 * J, 32 * kk, lane);
                lbJ[J] = *reinterpret_cast<const f32x4 *>(&sm.TR[m3].lb[16 * J + 4 * q4]);
                if constexpr (RAW) rkJ[J] = *reinterpret_cast<const f32x4 *>(&sm.TR[m3].rk[16 * J + 4 * q4]);
            }
            const float lbr = sm.TR[m3].lb[16 * RB + l15];
            __builtin_amdgcn_sched_barrier(0);   // every LDS read of the step in flight at once
            float ebr = __builtin_amdgcn_exp2f(lbr), iq = 1.f;
            if constexpr (RAW) {
                // 1/|q_r| for the lane's row: its 8 KD values, then the four
                // lanes (q4) that share the row
                float ss = 0.f;
#pragma unroll
                for (int kk = 0; kk < KD; ++kk)
#pragma unroll
                    for (int u = 0; u < 8; ++u) ss = __builtin_fmaf((float)Qr[kk][u], (float)Qr[kk][u], ss);
                ss = swap_sum32(swap_sum16(ss));
                iq = inv_norm(ss);
                ebr *= iq;
            }
            // diag(e^b) Q S^T (S entering chunk c)
#pragma unroll
            for (int ob = 0; ob < 2; ++ob) {
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) x = mfma32(As[ob][kk], Qr[kk], x);
                QSp[ob] = x * ebr;
            }
            // P: K_J Q_RB^T gives lane s = 16 J + 4 q4 + e, r = 16 RB + l15,
            // and P[r][s] = e^{b_r - b_s} q_r.k_s for s <= r (the factor is
            // formed from the difference, so it is at most 1; the entries
            // above the diagonal are selected away, not multiplied)
            f32x4 pv[RB + 2];
#pragma unroll
            for (int J = 0; J <= RB; ++J) {
                f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) p = mfma32(Kj[J][kk], Qr[kk], p);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v = __builtin_amdgcn_exp2f(lbr - lbJ[J][e]) * p[e];
                    if constexpr (RAW) v *= rkJ[J][e] * iq;
                    pv[J][e] = (J < RB || 4 * q4 + e <= l15) ? v : 0.f;
                }
            }
            pv[RB + 1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k2 = 0; k2 < NP2; ++k2) Pp[k2] = acc_pair(pv[2 * k2], pv[2 * k2 + 1]);
        };
        QSp[0] = QSp[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k2 = 0; k2 < NP2; ++k2) Pp[k2] = bf16x8{};
        __syncthreads();
        int m3 = 0;                           // c mod 3
        for (long long c = 0; c < nhalf; c += 2) {
            o_step(c);
            qp_step(c, m3);
            m3 = m3 == 2 ? 0 : m3 + 1;
            __syncthreads();
            o_step(c + 1);
            qp_step(c + 1, m3);
            m3 = m3 == 2 ? 0 : m3 + 1;
            __syncthreads();
        }
    };
    if (w == 2)      out_loop(std::integral_constant<int, 0>{});
    else if (w == 3) out_loop(std::integral_constant<int, 1>{});
    else if (w == 7) out_loop(std::integral_constant<int, 2>{});
    else             out_loop(std::integral_constant<int, 3>{});
}

// First chunk of every packed sequence: base[n] = sum over m < n of
// ceil(len_m / C), base[N] = the total.  One workgroup: each thread sums a
// run of consecutive sequences, then an exclusive scan over the 256 runs.
__global__ __launch_bounds__(256) void chunk_base_kernel(const int32_t *cu, int N, int32_t *base) {
    __shared__ int part[256];
    const int t = threadIdx.x;
    const int per = (N + 255) / 256;
    const int m0 = t * per < N ? t * per : N;
    const int m1 = m0 + per < N ? m0 + per : N;
    int s = 0;
    for (int m = m0; m < m1; ++m) s += (cu[m + 1] - cu[m] + C - 1) / C;
    part[t] = s;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {   // inclusive scan (Hillis-Steele)
        const int x = t >= d ? part[t - d] : 0;
        __syncthreads();
        part[t] += x;
        __syncthreads();
    }
    int acc = part[t] - s;                // exclusive
    for (int m = m0; m < m1; ++m) {
        base[m] = acc;
        acc += (cu[m + 1] - cu[m] + C - 1) / C;
    }
    if (t == 255) base[N] = part[255];
}

}  // namespace

hipError_t launch_chunk_base(const int32_t *cu_seqlens, int N, int32_t *chunk_base,
                             hipStream_t s) {
    if (N < 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(chunk_base_kernel, dim3(1), dim3(256), 0, s, cu_seqlens, N, chunk_base);
    return hipGetLastError();
}

hipError_t launch_prefill_chain(int D, const PrefillArgs &a, hipStream_t s) {
    const long long units = (long long)a.N * a.H;
    if (units <= 0) return hipSuccess;
    if (a.cu_seqlens) {
        hipLaunchKernelGGL(chunk_base_kernel, dim3(1), dim3(256), 0, s, a.cu_seqlens, a.N,
                           a.chunk_base);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long long prep_units = a.max_chunks * a.H;
    if (prep_units > 0) {
        dim3 grid((unsigned)((prep_units + 7) / 8 * 8)), block(256);
        if (a.xg) {
            if (D == 128) hipLaunchKernelGGL((prep_kernel<128, true>), grid, block, 0, s, a);
            else          hipLaunchKernelGGL((prep_kernel<64, true>), grid, block, 0, s, a);
        } else {
            if (D == 128) hipLaunchKernelGGL((prep_kernel<128, false>), grid, block, 0, s, a);
            else          hipLaunchKernelGGL((prep_kernel<64, false>), grid, block, 0, s, a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int ntile = D / BV;
    const long long blocks = ((units + 7) / 8) * 8 * ntile;
    dim3 grid((unsigned)blocks), block(512);
    if (a.xg) {
        if (D == 128) hipLaunchKernelGGL((chain_kernel<128, true>), grid, block, 0, s, a);
        else          hipLaunchKernelGGL((chain_kernel<64, true>), grid, block, 0, s, a);
    } else {
        if (D == 128) hipLaunchKernelGGL((chain_kernel<128, false>), grid, block, 0, s, a);
        else          hipLaunchKernelGGL((chain_kernel<64, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace gdr
