// Causal paged attention for many query rows per sequence (long prefill
// chunks): the rows of one (sequence, KV head) in blocks of 128, with the
// sequence's keys and values staged through LDS once per work-group and
// shared by its four waves.
//
// What is computed is the multi-token rule of paged_multi_token_attention:
// the n query rows of sequence s are its last n tokens, row i at position
// L - n + i attends positions 0 .. L - n + i, through the block table as in
// decode (cache-structure page, "软件地址翻译"; chunked prefill on the
// "vLLM 核心工程深度剖析" page, section 6.1).
//
// How it maps onto CDNA4:
//  * Work-group (KV head, row block, sequence), 4 waves, 32 rows per wave as
//    two 16-row MFMA tiles; a row is a (query token, group member) pair.
//  * The keys and values are walked in 32-token units staged in LDS, one
//    barrier per unit.  bf16 pools: four stages, filled by direct
//    global-to-LDS loads (global_load_lds_dwordx4: lane i of a wave
//    instruction lands at base + 16 i) issued three units ahead, so no
//    registers hold data in flight; the loop is software-pipelined: a
//    unit's softmax (vector work) comes first, then one run of matrix work,
//    its value sums and the scores of the next unit, which the other wave on
//    the SIMD overlaps with its own softmax.  FP8 pools: two
//    stages, the next unit's codes loaded into registers and converted to
//    bf16 on the way into LDS.
//    Keys sit in LDS as [hs/8][32 positions] 16-byte chunks, so a lane's
//    16-byte read is the A operand of v_mfma_f32_16x16x32_bf16 (position
//    row c, 8 head dims) and a lane group reads 256 contiguous bytes.
//    Position 16 mp + m holds token key_token(16 mp + m) = 8 (m / 4) + 4 mp
//    + m % 4: the scores of M-tiles mp = 0, 1 then give lane group r the
//    tokens 8r .. 8r+7 in order, which is the token order of the value MFMA's
//    operands, so the probabilities need no exchange between lanes.  Values sit
//    as [hs][32 tokens] in four 16-byte slots per row, the slots of row d
//    permuted (vslot) so that the value-operand reads are free of bank
//    conflicts.
//  * Each wave reads one unit's key and value operands once from LDS and
//    uses them for both of its row tiles (scores, then the value sum with
//    hi + lo bf16 probability parts as in decode).
//  * Causal: a lane's row has its own limit; a wave stops computing at its
//    last row's limit, and the work-group stops loading at its last row's.
//  * The K/V loads use the caches normally: the other row blocks of the same
//    (sequence, KV head) read the same tiles.
//  * The block IDs of 64 consecutive blocks sit one per lane and each thread
//    fetches the one it needs with ds_bpermute; the next 64 are loaded while
//    the current ones are in use.  An ID outside the pool reads block 0 and
//    its tokens are masked (the same rule as decode).
#include <type_traits>

#include "attn_common.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kPfTiles = 2;                       // 16-row MFMA tiles per wave
constexpr int kPfRows = kPfWaves * kPfTiles * 16; // rows per work-group
constexpr int kPfUnit = 32;                       // tokens per staged unit

// The token whose key sits at LDS key position pos of a unit (see above).
__device__ __forceinline__ int key_token(int pos)
{
    return 8 * ((pos & 15) >> 2) + 4 * (pos >> 4) + (pos & 3);
}
// LDS slot (16 bytes) of tokens 8q .. 8q+7 of value row d: four slots per
// row, permuted by (d / 4) % 4 through 0, 3, 2, 1.  A value-operand read has
// lane group r = lane / 16 read slot r of row 16 i + lane % 16.  gfx950 serves
// a 128-bit LDS read in four cycles when no two lanes of a cycle share a
// 16-byte bank group; measured with the bank-conflict counter, this
// permutation keeps the value-operand read at that rate, while the plain
// layout, or the permutations q ^ ((d / 4) % 4) and 0, 3, 1, 2, cost four
// extra cycles per read.
__device__ __forceinline__ int vslot(int d, int q)
{
    return 4 * d + (q ^ ((0x6C >> (2 * ((d >> 2) & 3))) & 3));
}
constexpr int kXcds = 8;                          // MI355X: 8 XCDs of 32 compute units

template <int HS>
struct PfStage {
    bf16x8 k[HS / 8][kPfUnit];        // chunk f (head dims 8f .. 8f+7) of token t
    bf16x8 v[HS * 4];                 // slot vslot(d, q): head dim d, tokens 8q .. 8q+7
};

// s_waitcnt with vmcnt(n) and the other counters left alone (gfx9
// encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int n>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Global reads of one unit from FP8 pools: 2 * HS key and 2 * HS value
// pieces of 16 codes; a thread takes pieces tid, tid + 256, ...
template <int HS>
struct PfPieces {
    static constexpr int P = 2 * HS;  // pieces of each kind
    static constexpr int N = (P + kPfThreads - 1) / kPfThreads;
    u32x4 k[N];
    u32x4 v[N];
};

// 16 E4M3 codes to 16 bf16 (two 16-byte halves, codes 0-7 and 8-15).
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4& w, u32x4& lo, u32x4& hi)
{
    unsigned e[8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        fp8x4_to_bf16(w[i], e[2 * i], e[2 * i + 1]);
    lo = (u32x4){e[0], e[1], e[2], e[3]};
    hi = (u32x4){e[4], e[5], e[6], e[7]};
}

template <int HS, int BS, bool F8>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2))) void paged_prefill_kernel(
    const __bf16* __restrict__ q, const typename std::conditional<F8, uint8_t, __bf16>::type* __restrict__ k_cache,
    const typename std::conditional<F8, uint8_t, __bf16>::type* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ q_start, int32_t num_q_rows, int32_t max_q_len, int32_t Hq, int32_t Hkv, int32_t M,
    int32_t num_blocks, int32_t RB, float qscale, float oscale, void* __restrict__ out, int32_t out_f32,
    int32_t num_seqs, const int32_t* __restrict__ sched_order)
{
    static_assert(BS >= 16 && (BS % 16) == 0, "blocks of 16, 32 or 64 tokens");
    constexpr int TILE = HS * BS;  // elements of one (block, KV head) tile
    // LDS stages of 16-byte slots: keys [hs/8][32] first, then values
    constexpr int NST = F8 ? 2 : 4;
    constexpr int STAGE_SLOTS = F8 ? (int)(sizeof(PfStage<HS>) / 16) : HS * 8;
    constexpr int KSLOTS = HS * 4;
    __shared__ bf16x8 lds[NST * STAGE_SLOTS];

    // Work order.  Work-groups are dealt to the 8 XCDs round-robin by their
    // linear index p (XCD p % 8), each XCD has its own L2, and on an XCD
    // they start in increasing p.  The RB row blocks of one (sequence, KV
    // head) pair read the same keys and values, so they go to one XCD: pair
    // g = rank * Hkv + kvh runs on XCD g % 8, its row blocks at consecutive
    // slots p / 8 there.  Pairs are taken in rank order, the sequence of
    // rank y being sched_order[y] (longest first, from the longest-first
    // schedule) or sequence y without one, and a pair's row blocks last row
    // block first (it sees the most tokens): so the longest work starts
    // first on every XCD and no long sequence is left running alone at the
    // end.  The grid is rounded up to whole rounds of 8 pairs; work-groups
    // past the last pair exit at once.
    const int64_t p = blockIdx.x;
    const int64_t xcd = p % kXcds, slot = p / kXcds;
    const int64_t pair = (slot / RB) * kXcds + xcd;
    if (pair >= (int64_t)num_seqs * Hkv)
        return;  // uniform, before any barrier
    const int rb = RB - 1 - (int)(slot % RB);
    const int kvh = (int)(pair % Hkv);
    const int rank = (int)(pair / Hkv);
    int s = sched_order ? sched_order[rank] : rank;
    // an order that does not belong to this batch (caller error) names a
    // sequence outside it: that work-group writes nothing
    const bool s_ok = (unsigned)s < (unsigned)num_seqs;
    s = s_ok ? s : 0;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane >> 4;
    const int c = lane & 15;
    const int G = Hq / Hkv;

    int qs0 = q_start[s];
    const int qs1 = q_start[s + 1];
    int n = qs1 - qs0;
    if (qs0 < 0 || n < 0 || qs1 > num_q_rows || !s_ok)
        n = 0;
    n = n < max_q_len ? n : max_q_len;
    const int nrows = n * G;
    const int row0 = rb * kPfRows;
    if (row0 >= nrows)
        return;  // uniform, before any barrier
    const int L_in = seq_lens[s];
    const int L = L_in < 0 ? 0 : (L_in > M * BS ? M * BS : L_in);
    auto out_row = [&](int rho) __attribute__((always_inline)) -> int64_t {
        const int i = rho / G;
        return ((int64_t)(qs0 + i) * Hq + (int64_t)kvh * G + (rho - i * G)) * HS;
    };
    const int last_row = (row0 + kPfRows < nrows ? row0 + kPfRows : nrows) - 1;
    if (L == 0) {
        for (int idx = tid; idx < (last_row - row0 + 1) * HS; idx += kPfThreads)
            store_out<__bf16>(out, out_row(row0 + idx / HS) + idx % HS, 0.f, out_f32);
        return;
    }
    // row rho sees the tokens below L - n + rho / G + 1 (at least 0)
    auto limit = [&](int rho) __attribute__((always_inline)) {
        const int v = L - n + rho / G + 1;
        return v < 0 ? 0 : v;
    };
    const int L_wg = limit(last_row);                     // this work-group's last token + 1
    const int nunits = (L_wg + kPfUnit - 1) / kPfUnit;
    const int wrow0 = row0 + w * kPfTiles * 16;           // this wave's first row
    const int wlast = (wrow0 + kPfTiles * 16 < nrows ? wrow0 + kPfTiles * 16 : nrows) - 1;
    const int L_w = wrow0 < nrows ? limit(wlast) : 0;     // this wave computes tokens below L_w

    // query operands and per-lane row limits of the two tiles; padding rows
    // repeat a real row and are never stored
    bf16x8 qr[kPfTiles][HS / 32];
    int Lq[kPfTiles];
    int Lmin[kPfTiles];
#pragma unroll
    for (int kt = 0; kt < kPfTiles; ++kt) {
        const int tb = wrow0 + kt * 16;
        const int rho = (tb + c) % nrows;
        Lq[kt] = limit(rho);
        Lmin[kt] = limit(tb < nrows ? tb : nrows - 1);
        const __bf16* qh = q + out_row(rho);
#pragma unroll
        for (int i = 0; i < HS / 32; ++i)
            qr[kt][i] = *(const bf16x8*)(qh + 32 * i + 8 * r);
    }

    f32x4 O[kPfTiles][HS / 16];
    // m_thr: the raw score above which the running maximum is raised,
    // (m_run + kRescaleSlack) / qscale, kept beside m_run so that the test
    // per unit is one compare
    float m_run[kPfTiles], m_thr[kPfTiles], l_part[kPfTiles];
#pragma unroll
    for (int kt = 0; kt < kPfTiles; ++kt) {
        m_run[kt] = -1e30f;
        m_thr[kt] = (-1e30f + kRescaleSlack) / qscale;
        l_part[kt] = 0.f;
#pragma unroll
        for (int i = 0; i < HS / 16; ++i)
            O[kt][i] = (f32x4)0.f;
    }

    // ---- FP8 register path: block IDs in a window of 64 table entries, one per lane ----
    const int32_t* trow = block_tables + (int64_t)s * M;
    // (register path only; the bf16 path reads table entries with scalar loads)
    int win = 0;
    int32_t ids = 0, ids_next = 0;
    if constexpr (F8) {
        ids = lane < M ? trow[lane] : 0;
        ids_next = 64 + lane < M ? trow[64 + lane] : 0;
    }
    const int64_t head_off = (int64_t)kvh * TILE;
    const int64_t block_stride = (int64_t)Hkv * TILE;
    // offset of table entry j (inside the window) in the pool, block 0 when
    // the ID is outside the pool
    auto block_at = [&](int j) __attribute__((always_inline)) -> int64_t {
        const int32_t id = __shfl(ids, j - win);
        return ((uint32_t)id < (uint32_t)num_blocks ? id : 0) * block_stride + head_off;
    };

    // ---- FP8 staging: this thread's pieces of unit u ----
    PfPieces<HS> pc;
    // Key piece p: chunk f16 = p / 32 (16 head dims) at LDS position p % 32.
    // Value piece p: head dim d = p % HS, tokens 16 h .. 16 h + 15 with
    // h = p / HS, so that the lanes of a wave deposit consecutive rows (the
    // deposits then hit distinct bank groups in every pass, as the reads do).
    auto fetch = [&](int u) __attribute__((always_inline)) {
        if constexpr (F8) {
            const int t0 = u * kPfUnit;
            if (t0 / BS >= win + 64) {  // uniform: the unit's first block left the window
                win += 64;
                ids = ids_next;
                ids_next = win + 64 + lane < M ? trow[win + 64 + lane] : 0;
            }
#pragma unroll
            for (int k = 0; k < PfPieces<HS>::N; ++k) {
                const int p = tid + k * kPfThreads;
                if (PfPieces<HS>::P % kPfThreads != 0 && p >= PfPieces<HS>::P)
                    break;
                const int f16 = p / kPfUnit, t = p % kPfUnit;  // LDS position t
                const int T = t0 + key_token(t);
                pc.k[k] = *(
                    (const u32x4*)(k_cache + block_at(T / BS) + ((int64_t)f16 * BS + T % BS) * 16));
                const int d = p % HS, h = p / HS;
                const int Tv = t0 + 16 * h;
                pc.v[k] = *(
                    (const u32x4*)(v_cache + block_at(Tv / BS) + (int64_t)d * BS + Tv % BS));
            }
        }
    };
    auto deposit = [&](PfStage<HS>& st) __attribute__((always_inline)) {
        if constexpr (F8) {
#pragma unroll
            for (int k = 0; k < PfPieces<HS>::N; ++k) {
                const int p = tid + k * kPfThreads;
                if (PfPieces<HS>::P % kPfThreads != 0 && p >= PfPieces<HS>::P)
                    break;
                const int f16 = p / kPfUnit, t = p % kPfUnit;
                u32x4 lo, hi;
                fp8x16_to_bf16(pc.k[k], lo, hi);
                st.k[2 * f16][t] = __builtin_bit_cast(bf16x8, lo);
                st.k[2 * f16 + 1][t] = __builtin_bit_cast(bf16x8, hi);
                const int d = p % HS, h = p / HS;
                fp8x16_to_bf16(pc.v[k], lo, hi);
                st.v[vslot(d, 2 * h)] = __builtin_bit_cast(bf16x8, lo);
                st.v[vslot(d, 2 * h + 1)] = __builtin_bit_cast(bf16x8, hi);
            }
        }
    };
    // tokens of unit u whose block ID is inside the pool (bit t: token 32u + t)
    auto unit_mask = [&](int u) __attribute__((always_inline)) -> unsigned {
        const uint64_t valid = __ballot((uint32_t)ids < (uint32_t)num_blocks);
        if constexpr (BS >= kPfUnit) {
            return ((valid >> ((u * kPfUnit) / BS - win)) & 1) ? 0xFFFFFFFFu : 0u;
        } else {
            const int j = (u * kPfUnit) / BS - win;  // two blocks of 16
            return (((valid >> j) & 1) ? 0x0000FFFFu : 0u) | (((valid >> (j + 1)) & 1) ? 0xFFFF0000u : 0u);
        }
    };

    // Scores of both row tiles for the unit whose keys are staged at kst, one
    // key M-tile (16 tokens) at a time.
    auto scores = [&](const bf16x8* kst, f32x4 (&S)[kPfTiles][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int mp = 0; mp < 2; ++mp) {
            bf16x8 kop[HS / 32];
#pragma unroll
            for (int i = 0; i < HS / 32; ++i)
                kop[i] = kst[(4 * i + r) * kPfUnit + 16 * mp + c];
#pragma unroll
            for (int kt = 0; kt < kPfTiles; ++kt) {
                S[kt][mp] = (f32x4)0.f;
#pragma unroll
                for (int i = 0; i < HS / 32; ++i)
                    S[kt][mp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[i], qr[kt][i], S[kt][mp], 0, 0, 0);
            }
        }
    };

    // Softmax and value sum of unit u from its scores S and the values staged
    // at vst.  With next_tag true it also forms the next unit's scores Sn
    // from the keys at kst_next: those matrix instructions do not depend on
    // this unit's vector work, and are issued with the value sums, after it.
    auto finish = [&](auto next_tag, const bf16x8* vst, const bf16x8* kst_next, int u, unsigned tmask,
                      const f32x4 (&S)[kPfTiles][2], f32x4 (&Sn)[kPfTiles][2]) __attribute__((always_inline)) {
        constexpr bool NEXT = decltype(next_tag)::value;
        const int t0 = u * kPfUnit;
        bf16x8 vop[HS / 16];
#pragma unroll
        for (int i = 0; i < HS / 16; ++i) {
            const int d = 16 * i + c;
            vop[i] = vst[vslot(d, r)];
        }
        bf16x8 kop[2][HS / 32];
        if constexpr (NEXT) {
#pragma unroll
            for (int mp = 0; mp < 2; ++mp)
#pragma unroll
                for (int i = 0; i < HS / 32; ++i)
                    kop[mp][i] = kst_next[(4 * i + r) * kPfUnit + 16 * mp + c];
        }
        const bool all_valid = tmask == 0xFFFFFFFFu;
        // raw scores; the scale is applied inside the exponent (qscale > 0
        // keeps the maximum where it is)
        float sc[kPfTiles][8];
#pragma unroll
        for (int kt = 0; kt < kPfTiles; ++kt)
#pragma unroll
            for (int mp = 0; mp < 2; ++mp)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    sc[kt][4 * mp + jj] = S[kt][mp][jj];
        if (t0 + kPfUnit > Lmin[0] || t0 + kPfUnit > Lmin[1] || !all_valid) {
            // a real branch: most units need no masking.  Token tt = 8r + e
            // of the unit (e = 4mp + jj, key_token order) is kept when e is
            // below lim = Lq - t0 - 8r and bit e of tm = tmask >> 8r is set;
            // the asm keeps lim and tm from being formed before the branch
            int tm = (int)(tmask >> (8 * r));
            asm volatile("" : "+v"(tm));
#pragma unroll
            for (int kt = 0; kt < kPfTiles; ++kt) {
                int lim = Lq[kt] - t0 - 8 * r;
                asm volatile("" : "+v"(lim));
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    sc[kt][e] = (e < lim && ((tm >> e) & 1)) ? sc[kt][e] : -INFINITY;
            }
        }
        // Online softmax of tile kt, in two parts.  raise_max: the running
        // maximum is raised only when a score exceeds it by more than
        // kRescaleSlack, and then alpha (the factor the accumulators are
        // rescaled by, in rescale_tile, before the next value sum into them)
        // is formed; probs: the exponentials and the bf16 hi / lo probability
        // operands.
        auto raise_max = [&](int kt, float& alpha) __attribute__((always_inline)) -> bool {
            // IEEE maximum (NaN-propagating): three-operand instructions
            // that need no canonicalization of the matrix results, unlike fmaxf
            // (grouped so that it forms four instructions: three of three
            // operands and one of two)
            const float m1 = __builtin_elementwise_maximum(
                __builtin_elementwise_maximum(sc[kt][0], sc[kt][1]), sc[kt][2]);
            const float m2 = __builtin_elementwise_maximum(
                __builtin_elementwise_maximum(sc[kt][3], sc[kt][4]), sc[kt][5]);
            const float m3 = __builtin_elementwise_maximum(
                __builtin_elementwise_maximum(sc[kt][6], sc[kt][7]), m1);
            const float mx = __builtin_elementwise_maximum(m2, m3);
            // A row's maximum exceeds the running maximum by the slack exactly
            // when one of its lanes' own maxima does (the running maximum is
            // the same in the row's four lane groups, and scaling by qscale > 0
            // keeps the order), so the ballot needs no exchange between lane
            // groups; the row maximum is formed only when the maximum rises.
            const bool raise = __ballot(mx > m_thr[kt]) != 0;  // uniform
            alpha = 1.f;
            if (raise) {
                const float m_new = fmaxf(m_run[kt], max_over_lane_groups(mx) * qscale);
                alpha = __builtin_amdgcn_exp2f(m_run[kt] - m_new);
                m_run[kt] = m_new;
                m_thr[kt] = (m_new + kRescaleSlack) / qscale;
                l_part[kt] *= alpha;
            }
            return raise;
        };
        auto probs = [&](int kt, bf16x8& hi, bf16x8& lo) __attribute__((always_inline)) {
            const float m_cur = m_run[kt];
            float pv[8];  // pv[e]: token 8r + e (key_token order)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kt][e], qscale, -m_cur));
                l_part[kt] += pv[e];
            }
            // hi = bf16(p) two at a time; lo = bf16(p - hi), with hi read back
            // from the packed pair by shifts (exact)
            u32x4 hw, lw;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f32x2 pp = {pv[2 * e], pv[2 * e + 1]};
                const unsigned hb = __builtin_bit_cast(unsigned, __builtin_convertvector(pp, bf16x2));
                const f32x2 rem = {pp[0] - __builtin_bit_cast(float, hb << 16),
                                   pp[1] - __builtin_bit_cast(float, hb & 0xFFFF0000u)};
                hw[e] = hb;
                lw[e] = __builtin_bit_cast(unsigned, __builtin_convertvector(rem, bf16x2));
            }
            hi = __builtin_bit_cast(bf16x8, hw);
            lo = __builtin_bit_cast(bf16x8, lw);
        };
        auto rescale_tile = [&](int kt, float alpha) __attribute__((always_inline)) {
            float a_row[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                a_row[jj] = __shfl(alpha, 4 * r + jj);
#pragma unroll
            for (int i = 0; i < HS / 16; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    O[kt][i][jj] *= a_row[jj];
        };
        auto value_sum = [&](int kt, const bf16x8& hi, const bf16x8& lo) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < HS / 16; ++i)
                O[kt][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, vop[i], O[kt][i], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < HS / 16; ++i)
                O[kt][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, vop[i], O[kt][i], 0, 0, 0);
        };
        // Every rare branch (raise and rescale of both tiles, value masking)
        // comes first, so that what follows is one straight run.
        float a0, a1;
        if (raise_max(0, a0))
            rescale_tile(0, a0);
        if (raise_max(1, a1))
            rescale_tile(1, a1);
        if (t0 + kPfUnit > L || !all_valid) {
            // value slots past the sequence or in a skipped block may hold
            // anything: zero them so that 0 * NaN never reaches the sum
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int tt = 8 * r + e;
                const bool keep = t0 + tt < L && ((tmask >> tt) & 1);
#pragma unroll
                for (int i = 0; i < HS / 16; ++i)
                    vop[i][e] = keep ? vop[i][e] : (__bf16)0.f;
            }
        }
        bf16x8 hi0, lo0, hi1, lo1;
        if constexpr (NEXT) {
            // Two phases: every exponential of the unit first, then every
            // matrix instruction (the next unit's scores and this unit's value
            // sums) at raised wave priority.  A wave issues an MFMA and the
            // vector instructions after it almost one after the other, so the
            // overlap comes from the other wave on the SIMD: the one with
            // matrix work ready issues it first while the other computes its
            // softmax.
            probs(0, hi0, lo0);
            probs(1, hi1, lo1);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int mp = 0; mp < 2; ++mp)
#pragma unroll
                for (int kt = 0; kt < kPfTiles; ++kt) {
                    Sn[kt][mp] = (f32x4)0.f;
#pragma unroll
                    for (int i = 0; i < HS / 32; ++i)
                        Sn[kt][mp] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[mp][i], qr[kt][i], Sn[kt][mp], 0, 0, 0);
                }
            value_sum(0, hi0, lo0);
            value_sum(1, hi1, lo1);
            __builtin_amdgcn_s_setprio(0);
        } else {
            // tile 0's value sum with tile 1's exponentials written next to it
            probs(0, hi0, lo0);
            __builtin_amdgcn_s_setprio(1);
            value_sum(0, hi0, lo0);
            probs(1, hi1, lo1);
#pragma unroll
            for (int k = 0; k < 2 * (HS / 16); ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four vector instructions
            }
            value_sum(1, hi1, lo1);
            __builtin_amdgcn_s_setprio(0);
        }
    };
    auto compute = [&](const bf16x8* kst, const bf16x8* vst, int u, unsigned tmask) __attribute__((always_inline)) {
        f32x4 S[kPfTiles][2];
        scores(kst, S);
        finish(std::false_type(), vst, nullptr, u, tmask, S, S);
    };

    // ---- the unit loop: fetch u+1 while computing u, one barrier per unit ----
    if constexpr (F8) {
        // ---- register staging: fetch u+1 while computing u ----
        PfStage<HS>* stage = reinterpret_cast<PfStage<HS>*>(lds);
        fetch(0);
        unsigned mask_cur = unit_mask(0);
        deposit(stage[0]);
        __syncthreads();
        for (int u = 0; u < nunits; ++u) {
            unsigned mask_next = 0;
            if (u + 1 < nunits) {
                fetch(u + 1);
                mask_next = unit_mask(u + 1);
            }
            if (u * kPfUnit < L_w)  // uniform per wave: this wave's rows see some of the unit
                compute(&stage[u & 1].k[0][0], lds + (u & 1) * STAGE_SLOTS + KSLOTS, u, mask_cur);
            if (u + 1 < nunits)
                deposit(stage[(u + 1) & 1]);
            mask_cur = mask_next;
            __syncthreads();
        }
    } else {
        // ---- direct global-to-LDS loads, three units ahead, four stages ----
        // This thread's slots: key slot p = tid + 256 k is chunk p / 32 at
        // position p % 32 = tid % 32, token key_token(tid % 32); value slot p
        // = vslot(d, q8) is row d = p / 4, holding tokens 8 q8 .. 8 q8 + 7,
        // where q8 depends on p % 4 and (d / 4) % 4 = (tid / 16) % 4 only: the
        // same q8 for every k.
        constexpr int NP = (4 * HS) / kPfThreads;  // slots of each kind per thread
        constexpr int NDMA = 2 * NP;               // load instructions per wave per unit
        const int tK = key_token(tid % kPfUnit);
        const int q8 = (tid & 3) ^ ((0x6C >> (2 * ((tid >> 4) & 3))) & 3);  // vslot(tid / 4, q8) = tid
        // Block IDs: a unit spans at most two table entries, j0 = 32 v / BS
        // and j0 + 1 (B = 16), read with scalar loads (uniform addresses) one
        // unit before the unit's loads are issued; each lane takes the entry
        // of its key token and of its value tokens.  Entries past the row are
        // read at its last index (their tokens are past the sequence).
        auto entries = [&](int v, int32_t& e0, int32_t& e1) __attribute__((always_inline)) {
            const int j0 = (v * kPfUnit) / BS;
            e0 = trow[j0 < M ? j0 : M - 1];
            e1 = trow[j0 + 1 < M ? j0 + 1 : M - 1];
        };
        auto base_of = [&](int32_t id) __attribute__((always_inline)) -> int64_t {
            return ((uint32_t)id < (uint32_t)num_blocks ? id : 0) * block_stride + head_off;
        };
        // loads of unit v into stage v % NST (every iteration issues them,
        // also past the last unit, into the free stage: a fixed count per
        // iteration for the waits below)
        // A unit starts a block (B <= 32) or half of one (B = 64), so which of
        // the two entries a lane's token uses, and its offset in the block up
        // to the unit's start, do not depend on the unit.
        const bool k_second = BS == 16 && tK >= 16, v_second = BS == 16 && q8 >= 2;
        const int k_off = (tK % BS) * 8, v_off = (8 * q8) % BS;
        auto issue = [&](int v, int32_t e0, int32_t e1) __attribute__((always_inline)) {
            __attribute__((address_space(3))) bf16x8* sb =
                (__attribute__((address_space(3))) bf16x8*)(lds + (v % NST) * STAGE_SLOTS);
            const int64_t b0 = base_of(e0), b1 = base_of(e1);  // uniform
            const int unit_off = (v * kPfUnit) % BS;           // 32 in the second half of a 64-token block
            const int64_t kb = (k_second ? b1 : b0) + k_off + unit_off * 8;
            const int64_t vb = (v_second ? b1 : b0) + v_off + unit_off;
#pragma unroll
            for (int k = 0; k < NP; ++k) {
                const int f = tid / kPfUnit + k * (kPfThreads / kPfUnit);
                const int d = tid / 4 + k * (kPfThreads / 4);
                const int slot = k * kPfThreads + w * 64;  // this wave's 64 slots
                __builtin_amdgcn_global_load_lds((const void*)(k_cache + kb + (int64_t)f * BS * 8), sb + slot, 16,
                                                 0, 0);
                __builtin_amdgcn_global_load_lds((const void*)(v_cache + vb + (int64_t)d * BS), sb + KSLOTS + slot,
                                                 16, 0, 0);
            }
        };
        // Software pipeline over units: in iteration u, unit u + 1 has landed
        // and its scores are formed while unit u's softmax and value sum run
        // (finish), so the loads run three units ahead into four stages.
        // Entries of units u (a), u+1 (b), u+2 (c), u+3 (d).
        int32_t a0, a1, b0, b1, c0, c1, d0, d1;
        entries(0, a0, a1);
        entries(1, b0, b1);
        entries(2, c0, c1);
        entries(3, d0, d1);
        issue(0, a0, a1);
        issue(1, b0, b1);
        issue(2, c0, c1);
        // the units this wave computes (its rows see tokens below L_w)
        const int nu_w = (L_w + kPfUnit - 1) / kPfUnit < nunits ? (L_w + kPfUnit - 1) / kPfUnit : nunits;
        f32x4 S[kPfTiles][2];
        wait_vmcnt<2 * NDMA>();  // loads(0) landed; loads(1), loads(2) may be outstanding
        __syncthreads();
        if (nu_w > 0)
            scores(lds, S);
        for (int u = 0; u < nunits; ++u) {
            // issued before this point, in order: ..., loads(u+1), loads(u+2).
            // This wave's loads of unit u+1 have landed once at most NDMA are
            // outstanding; the barrier makes every wave's part visible and
            // frees the stage of unit u-1
            wait_vmcnt<NDMA>();
            __syncthreads();
            int32_t e0, e1;
            entries(u + 4, e0, e1);
            issue(u + 3, d0, d1);
            // tokens of unit u whose block ID is inside the pool
            const bool ok0 = (uint32_t)a0 < (uint32_t)num_blocks, ok1 = (uint32_t)a1 < (uint32_t)num_blocks;
            const unsigned tmask = BS >= kPfUnit ? (ok0 ? 0xFFFFFFFFu : 0u)
                                                 : ((ok0 ? 0x0000FFFFu : 0u) | (ok1 ? 0xFFFF0000u : 0u));
            if (u < nu_w) {  // uniform per wave
                // the next unit's keys have landed (also past this wave's
                // last unit or the work-group's, where the scores go unused)
                f32x4 Sn[kPfTiles][2];
                finish(std::true_type(), lds + (u % NST) * STAGE_SLOTS + KSLOTS,
                       lds + ((u + 1) % NST) * STAGE_SLOTS, u, tmask, S, Sn);
#pragma unroll
                for (int kt = 0; kt < kPfTiles; ++kt)
#pragma unroll
                    for (int mp = 0; mp < 2; ++mp)
                        S[kt][mp] = Sn[kt][mp];
            }
            a0 = b0; a1 = b1; b0 = c0; b1 = c1; c0 = d0; c1 = d1; d0 = e0; d1 = e1;
        }
        // the last three iterations' loads still write LDS: wait before the
        // work-group's LDS can be handed to another
        wait_vmcnt<0>();
    }

    // ---- normalise and store the rows ----
#pragma unroll
    for (int kt = 0; kt < kPfTiles; ++kt) {
        float l_tot = l_part[kt] + __shfl_xor(l_part[kt], 16);
        l_tot += __shfl_xor(l_tot, 32);
        const int tb = wrow0 + kt * 16;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int g = 4 * r + jj;
            const float l_g = __shfl(l_tot, g);
            const float inv = l_g > 0.f ? oscale / l_g : 0.f;
            if (tb + g < nrows) {
                const int64_t dst = out_row(tb + g);
#pragma unroll
                for (int i = 0; i < HS / 16; ++i)
                    store_out<__bf16>(out, dst + 16 * i + c, O[kt][i][jj] * inv, out_f32);
            }
        }
    }
}

template <int HS, int BS, bool F8>
static hipError_t launch_prefill_typed(const DecodeArgs& a, hipStream_t stream)
{
    using C = typename std::conditional<F8, uint8_t, __bf16>::type;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int RB = (a.max_q_len * G + kPfRows - 1) / kPfRows;
    const float qscale = a.scale * kLog2e * (F8 ? a.k_scale : 1.0f);
    // whole rounds of kXcds (sequence, KV head) pairs (see the work order in the kernel)
    const int64_t pairs = (int64_t)a.num_seqs * a.num_kv_heads;
    const int64_t groups = (pairs + kXcds - 1) / kXcds * kXcds * RB;  // < 2^31: checked on the host
    hipLaunchKernelGGL((paged_prefill_kernel<HS, BS, F8>), dim3((unsigned)groups), dim3(kPfThreads), 0,
                       stream, (const __bf16*)a.q, (const C*)a.k_cache, (const C*)a.v_cache, a.block_tables,
                       a.seq_lens, a.q_start, a.num_q_rows, a.max_q_len, a.num_q_heads, a.num_kv_heads,
                       a.max_blocks_per_seq, a.num_blocks, RB, qscale, F8 ? a.v_scale : 1.0f, a.out, a.out_f32,
                       a.num_seqs, a.sched_order);
    return hipGetLastError();
}

template <int HS, bool F8>
static hipError_t launch_prefill_block(const DecodeArgs& a, hipStream_t stream)
{
    switch (a.block_size) {
    case 16: return launch_prefill_typed<HS, 16, F8>(a, stream);
    case 32: return launch_prefill_typed<HS, 32, F8>(a, stream);
    default: return launch_prefill_typed<HS, 64, F8>(a, stream);
    }
}

bool prefill_shape_supported(int32_t dtype, int32_t block_size, int32_t head_size)
{
    return (dtype == 1 || dtype == 2) && block_size >= 16 && (head_size == 64 || head_size == 128);
}

int64_t prefill_work_groups(int64_t num_seqs, int64_t num_q_heads, int64_t num_kv_heads, int64_t max_q_len)
{
    const int64_t G = num_q_heads / num_kv_heads;
    return (num_seqs * num_kv_heads + kXcds - 1) / kXcds * kXcds * ((max_q_len * G + kPfRows - 1) / kPfRows);
}

bool prefill_supported(const DecodeArgs& a)
{
    return prefill_shape_supported(a.dtype, a.block_size, a.head_size) && a.q_start != nullptr;
}

int64_t prefill_work_groups(const DecodeArgs& a)
{
    return prefill_work_groups(a.num_seqs, a.num_q_heads, a.num_kv_heads, a.max_q_len);
}

hipError_t launch_prefill(const DecodeArgs& a, hipStream_t stream)
{
    const bool f8 = a.dtype == 2;  // PKV_FP8_E4M3
    if (a.head_size == 128)
        return f8 ? launch_prefill_block<128, true>(a, stream) : launch_prefill_block<128, false>(a, stream);
    return f8 ? launch_prefill_block<64, true>(a, stream) : launch_prefill_block<64, false>(a, stream);
}

}  // namespace pkv
