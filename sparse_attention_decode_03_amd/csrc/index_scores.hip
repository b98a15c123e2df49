// index_scores.hip -- lightning-indexer scores on the gfx950 matrix cores.
//
// score[r, t] = sum_h w[r, h] * max(0, q_idx[r, h, :] . k_normed[s, t, :])
// (glm5next_dsa/layer.rs source page: module header trap list and the
// `weights_proj` field doc -- the head weights already carry
// index_heads^-0.5, the scorer adds no scale; `indexer_forward` -- the key
// cache is read token-major as k[raw * D + d]).
//
// Design (HBM-bound: 256 B of keys per token at D = 128 against 8 kflop):
//  - One workgroup walks every W-th tile of one sequence (256 tokens; 128
//    when two or four rows share the keys, or when the call has too few
//    tiles to give each workgroup more than one) and scores each tile for
//    the rows of its unit: all K rows of the sequence (the rows of a verify
//    share one key read), or a group of four (or two) of them when K is
//    larger, each group walking the keys on its own. Keys stream HBM -> VGPR with fully coalesced 16-byte
//    loads (the next tile's loads are in flight while the current tile
//    computes) and are parked in LDS with an XOR swizzle, then re-read in
//    matrix-core operand order without bank conflicts.
//  - The keys are read once, so their loads carry the non-temporal hint:
//    the stream then no longer evicts the scores this pass writes from L2,
//    whose dirty lines would otherwise reach HBM a few at a time in the
//    middle of the read stream (measured: 12 % of the pass).
//  - The contraction is a 32x32x16 bf16 MFMA with the (up to 32) index heads
//    as M and 32 tokens as N; D is the reduction. A lane ends with 16 head
//    partials of one token; ReLU, weight and head sum run in fp32 in a fixed
//    order and one cross-lane add finishes the token (deterministic).
//  - Optionally the pass also writes, for every row, the largest order key
//    of each aligned 4-token and 32-token group (cross-lane max of the
//    finished scores, two stores per 32 tokens). Selection draws its
//    threshold from these.
#include <type_traits>

#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kIdxThreads = 256; // 4 waves x 64 tokens of a tile
constexpr int kIdxWgTarget = 512; // workgroups the tiles of a call spread over

// LDS: the key tile, up to 256 tokens x 16 chunks of 16 bytes (64 KiB at D = 128).

// The epilogue of one 32-token block of one row from its 32x32 MFMA result
// (lane: token t, 16 head partials): ReLU-weighted head sum, the score store
// and (GM) the group maxima. srow, g4row and g32row point at the row's
// scores and group-maximum rows; t is the lane's token, L the row length.
template <bool GM>
__device__ __forceinline__ void block_epilogue(const float (&wv)[16], const floatx16 &acc, int lane,
                                               int t, int L, float *srow, uint32_t *g4row,
                                               uint32_t *g32row)
{
    // ReLU as a signed-integer max on the bits: a negative float (sign bit
    // set) compares below 0, so this is max(x, 0) for every non-NaN x (-0
    // gives +0) in one instruction; fmaxf would first quiet a possible
    // signalling NaN with an extra instruction per value
    float part = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; v++)
        part = __builtin_fmaf(wv[v], __int_as_float(max(__float_as_int(acc[v]), 0)), part);
    const float tot = add_xor32(part);
    const int hl = lane / 32;
    if (hl == 0 && t < L)
        srow[t] = tot;
    if (GM) {
        // groups are aligned: a quad of lanes holds a 4-token group, lanes
        // 0..31 the 32-token group
        uint32_t k = t < L ? score_key(tot) : 0u;
        k = max(k, dpp_u32<kDppQuadXor1>(k));
        k = max(k, dpp_u32<kDppQuadXor2>(k));
        if (hl == 0 && (lane & 3) == 0 && t < L)
            g4row[t >> 2] = k;
        k = max(k, dpp_u32<kDppRowHalfMirror>(k));
        k = max(k, dpp_u32<kDppRowMirror>(k)); // every lane: its row's max
        const uint32_t k32 = max((uint32_t)__builtin_amdgcn_readlane((int)k, 0),
                                 (uint32_t)__builtin_amdgcn_readlane((int)k, 16));
        if (lane == 0 && t < L)
            g32row[t >> 5] = k32;
    }
}

template <int D, bool ONE_ROW, bool GM, int TILE>
__global__ __launch_bounds__(kIdxThreads, 2) void k_index_scores(
    const uint16_t *__restrict__ q_idx, const float *__restrict__ w,
    const uint16_t *__restrict__ k_normed, const int32_t *__restrict__ seq_lens,
    float *__restrict__ scores, uint32_t *__restrict__ gm4, uint32_t *__restrict__ gm32, int S,
    int K, int KG, int Hi, int64_t cap, int max_len, int stride)
{
    constexpr int CH = D / 8;  // 16-byte chunks per key row
    constexpr int KS = D / 16; // MFMA k-steps
    // TILE tokens per tile: 256 or 128 (see rows_tile and row_tile)
    static_assert(TILE == 256 || TILE == 128, "tiles of 256 or 128 tokens");
    constexpr int LOADS = TILE * CH / kIdxThreads;
    __shared__ u32x4 lds[TILE * CH];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave); // uniform: scalar row math
    const int hl = lane / 32;

    // ---- balance the tiles of all units over about kIdxWgTarget workgroups
    // from the device-side lengths. A unit is KG rows of one sequence (all
    // K rows, or a group of them: unit u is rows KG (u mod RG) .. + KG - 1
    // of sequence u / RG, RG = K / KG). Every workgroup computes the same
    // split (tiles per workgroup from the total), unit u gets
    // ceil(tiles_u / tpw) workgroups, and this workgroup claims its unit and
    // slot from a prefix of those counts ----
    __shared__ uint32_t bscan[kIdxThreads / kWave + 1];
    __shared__ int claim[4];
    __shared__ int s_len[kMaxRowsPerSeq]; // lengths of the claimed unit's rows
    const int RG = K / KG;                // units per sequence
    const int SU = S * RG;                // units
    auto row_len = [&](int r) { return min(max(seq_lens[r], 0), max_len); };
    auto unit_row = [&](int u) { return (u / RG) * K + (u % RG) * KG; }; // the unit's first row
    auto seq_lmax = [&](int u) {
        int lm = 0;
        for (int j = 0; j < KG; j++)
            lm = max(lm, row_len(unit_row(u) + j));
        return lm;
    };
    const int per = (SU + kIdxThreads - 1) / kIdxThreads; // units per thread
    const int sq0 = min(tid * per, SU), sq1 = min(sq0 + per, SU);
    // the first unit's length is kept (the only one up to 256 units)
    const int lm0 = sq0 < sq1 ? seq_lmax(sq0) : 0;
    // Tiles that count for the split: a last tile of at most kIdxLightTail
    // tokens costs about one 32-token block and rides along with another
    // tile's workgroup (the interleave below hands it to one of them).
    auto tiles_of = [&](int lm) {
        const int nt = (lm + TILE - 1) / TILE;
        return (uint32_t)(nt > 1 && lm - (nt - 1) * TILE <= kIdxLightTail ? nt - 1 : nt);
    };
    uint32_t my_tiles = 0;
    for (int sq = sq0; sq < sq1; sq++)
        my_tiles += tiles_of(sq == sq0 ? lm0 : seq_lmax(sq));
    uint32_t total_tiles;
    (void)block_exclusive_scan<kIdxThreads>(my_tiles, bscan, &total_tiles);
    // Tiles per workgroup: the smallest count from ceil(total / target) up
    // whose split needs at most kIdxWgTarget workgroups (two per CU, all
    // resident at once), tried a few times; any count from the first on
    // needs at most kIdxWgTarget + SU workgroups, the grid.
    uint32_t tpw = max(1u, (total_tiles + kIdxWgTarget - 1) / kIdxWgTarget);
    uint32_t my_wgs, wg_base, total_wgs;
    for (int attempt = 0;; attempt++, tpw++) {
        my_wgs = 0;
        for (int sq = sq0; sq < sq1; sq++)
            my_wgs += (tiles_of(sq == sq0 ? lm0 : seq_lmax(sq)) + tpw - 1) / tpw;
        wg_base = block_exclusive_scan<kIdxThreads>(my_wgs, bscan, &total_wgs);
        if (total_wgs <= (uint32_t)kIdxWgTarget || attempt == 3)
            break;
    }
    if (tid == 0)
        claim[0] = -1;
    __syncthreads();
    const uint32_t me = blockIdx.x;
    if (me >= wg_base && me < wg_base + my_wgs) { // exactly one thread
        uint32_t at = wg_base;
        for (int sq = sq0; sq < sq1; sq++) {
            const int lm = sq == sq0 ? lm0 : seq_lmax(sq);
            const uint32_t w_s = (tiles_of(lm) + tpw - 1) / tpw;
            if (me < at + w_s) {
                claim[0] = sq;
                claim[1] = (int)(me - at);
                claim[2] = (int)w_s;
                claim[3] = lm;
                for (int j = 0; j < KG; j++)
                    s_len[j] = row_len(unit_row(sq) + j);
                break;
            }
            at += w_s;
        }
    }
    __syncthreads();
    // the claim is the same for every lane: read into scalar registers, so
    // that the key buffer's descriptor is scalar (a descriptor in vector
    // registers makes the compiler wrap every load in a loop over its
    // distinct values) and the tile loop branches on scalars
    const int unit = __builtin_amdgcn_readfirstlane(claim[0]);
    if (unit < 0)
        return; // past the last workgroup this split needs
    const int s = unit / RG;          // the unit's sequence
    const int rbase = unit_row(unit); // and its first row
    // the longest row of the unit: the tiles to score (from the claim, so
    // the first tile's loads go out with no further length load)
    const int lmax = __builtin_amdgcn_readfirstlane(claim[3]);
    // tiles interleave across the sequence's workgroups (workgroup x takes
    // tiles x, x + W, x + 2W, ...), so at any moment the workgroups stream
    // neighbouring tiles and spread over every HBM channel
    const int W = __builtin_amdgcn_readfirstlane(claim[2]);
    const int tile_first = __builtin_amdgcn_readfirstlane(claim[1]);
    const int tile_end = (lmax + TILE - 1) / TILE;
    if (tile_first >= tile_end)
        return;

    // The sequence's keys as a buffer resource whose range ends at the
    // longest row: the hardware returns zeros for loads past it, so the key
    // loads need no mask and no 64-bit address arithmetic. The whole offset
    // goes in the per-lane operand, the one the range check tests.
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(k_normed + (int64_t)s * cap * D), 0, lmax * D * 2, kBufferWord3);
    u32x4 regs[LOADS];
    // loads [I0, I1) of a tile's share of this thread: 16-byte piece
    // i * kIdxThreads + tid of the tile, i.e. row g / CH, chunk g % CH
    auto load_part = [&](int tile, auto i0c, auto i1c) {
        constexpr int I0 = decltype(i0c)::value, I1 = decltype(i1c)::value;
        const int tile_bytes = tile * TILE * D * 2;
#pragma unroll
        for (int i = I0; i < I1; i++)
            regs[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, tile_bytes + (i * kIdxThreads + tid) * 16,
                                                            0, kCachePolicyNT);
    };
    using IC0 = std::integral_constant<int, 0>;
    using ICH = std::integral_constant<int, LOADS / 2>;
    using ICL = std::integral_constant<int, LOADS>;
    // a tile's registers into LDS (XOR swizzle), half [I0, I1)
    auto park_part = [&](auto i0c, auto i1c) {
        constexpr int I0 = decltype(i0c)::value, I1 = decltype(i1c)::value;
#pragma unroll
        for (int i = I0; i < I1; i++) {
            const int g = i * kIdxThreads + tid;
            const int row = g / CH;
            const int c = g % CH;
            lds[row * CH + (c ^ (row & (CH - 1)))] = regs[i];
        }
    };

    // query operands: row (head) lane%32, k-chunks hl*KS + ks (the same k
    // order as the key operands); weights of the 16 heads this lane reduces
    const int h_row = lane & 31;
    bf16x8 qa[KS];
    float wv[16];
    // (branch-free: padding heads load head Hi-1 and are zeroed, so every
    // load of a row is in flight at once)
    auto load_row = [&](int r) {
        const uint16_t *qrow = q_idx + ((int64_t)r * Hi + min(h_row, Hi - 1)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            u32x4 v = *(const u32x4 *)(qrow + (hl * KS + ks) * 8);
            if (h_row >= Hi)
                v = u32x4{0u, 0u, 0u, 0u};
            qa[ks] = as_bf16x8(v);
        }
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int h = 8 * (v / 4) + 4 * hl + (v % 4);
            const float x = w[(int64_t)r * Hi + min(h, Hi - 1)];
            wv[v] = (h < Hi) ? x : 0.0f;
        }
    };

    // The epilogue of one 32-token block of row r.
    auto block_out = [&](int r, int L, int t0, int col0, const floatx16 &acc) {
        block_epilogue<GM>(wv, acc, lane, t0 + col0 + (lane & 31), L, scores + (int64_t)r * stride,
                           GM ? gm4 + (int64_t)r * (stride / 4) : nullptr,
                           GM ? gm32 + (int64_t)r * (stride / 32) : nullptr);
    };
    // One 32-token block: MFMA over D, then the epilogue.
    auto score_block = [&](int r, int L, int t0, int col0, const bf16x8 (&kb)[KS]) {
        floatx16 acc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            acc = mfma32x32x16(qa[ks], kb[ks], acc);
        block_out(r, L, t0, col0, acc);
    };
    // Two neighbouring blocks of one row: their MFMA chains interleaved, so
    // each product's latency hides behind the other chain (the arithmetic of
    // every element is that of score_block).
    // The key operands are read from LDS inside the k loop (the registers
    // also hold the next tile's loads).
    auto score_block_pair = [&](int r, int L, int t0, int col0) {
        floatx16 acc[2] = {};
        const int row0 = col0 + (lane & 31), row1 = row0 + 32;
        auto key = [&](int row, int ks) {
            const int c = hl * KS + ks;
            return as_bf16x8(lds[row * CH + (c ^ (row & (CH - 1)))]);
        };
        // operands of step ks + 1 requested before the products of step ks
        bf16x8 k0 = key(row0, 0), k1 = key(row1, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            bf16x8 n0 = k0, n1 = k1;
            if (ks + 1 < KS) {
                n0 = key(row0, ks + 1);
                n1 = key(row1, ks + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            acc[0] = mfma32x32x16(qa[ks], k0, acc[0]);
            acc[1] = mfma32x32x16(qa[ks], k1, acc[1]);
            __builtin_amdgcn_sched_barrier(0);
            k0 = n0;
            k1 = n1;
        }
        block_out(r, L, t0, col0, acc[0]);
        block_out(r, L, t0, col0 + 32, acc[1]);
    };

    // Several rows (KG > 1): the tile's KG x (TILE / 32) (row, block) items
    // are split into four contiguous ranges, one per wave, in row-major
    // order, so a wave keeps one row's query across blocks (with KG = 4 each
    // wave owns one row for the whole run and loads its query once).
    constexpr int kBlocks = TILE / 32;
    const int items = KG * kBlocks / (kIdxThreads / kWave);
    const int item0 = wave * items;
    // The first tile's key loads go out before the query's: the query is
    // used (padding heads zeroed) as soon as it lands, and loads issued
    // after it would wait for it.
    load_part(tile_first, IC0{}, ICL{});
    int loaded = -1;
    if (ONE_ROW) {
        load_row(rbase);
    } else if (item0 / kBlocks == (item0 + items - 1) / kBlocks) {
        loaded = item0 / kBlocks;
        load_row(rbase + loaded);
    }
    for (int tile = tile_first; tile < tile_end; tile += W) {
        const int t0 = tile * TILE;
        const bool more = tile + W < tile_end;
        __syncthreads(); // every wave is done reading the previous tile
        // park the tile in LDS half by half; each half's registers take the
        // next tile's loads at once, so the loads stay in flight while this
        // tile is parked and computed
        park_part(IC0{}, ICH{});
        if (more)
            load_part(tile + W, IC0{}, ICH{});
        park_part(ICH{}, ICL{});
        if (more)
            load_part(tile + W, ICH{}, ICL{});
        __syncthreads();

        if (ONE_ROW) {
            // wave w scores tokens [w TILE / 4, (w + 1) TILE / 4) of the tile:
            // NB 32-token blocks; key operands: column (token) lane%32,
            // k-chunks hl*KS + ks
            constexpr int NB = TILE / 128;
            bf16x8 kb[NB][KS];
#pragma unroll
            for (int b = 0; b < NB; b++) {
                const int row = wave * (TILE / 4) + b * 32 + (lane & 31);
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    const int c = hl * KS + ks;
                    kb[b][ks] = as_bf16x8(lds[row * CH + (c ^ (row & (CH - 1)))]);
                }
            }
#pragma unroll
            for (int b = 0; b < NB; b++)
                score_block(rbase, lmax, t0, wave * (TILE / 4) + b * 32, kb[b]);
        } else {
            // the wave's (row, 32-token block) items, two at a time: a range
            // starts at an even item and the blocks per row are even, so a
            // pair never straddles rows. Rows of one item range reuse the
            // loaded query. A pair runs when its first block is inside the
            // row (the second one's stores are masked past L).
            for (int it = item0; it < item0 + items; it += 2) {
                const int j = it / kBlocks;
                const int blk = it % kBlocks;
                const int r = rbase + j;
                // from LDS (no wait on the loads in flight), into a scalar
                const int L = __builtin_amdgcn_readfirstlane(s_len[j]);
                if (t0 + blk * 32 >= L)
                    continue;
                if (j != loaded) {
                    load_row(r);
                    loaded = j;
                }
                score_block_pair(r, L, t0, blk * 32);
            }
        }
    }
}

// Rows per unit of the K-row pass: K rows of a sequence are scored as K / KG
// units of KG rows, each walking the sequence's keys on its own (KG = 4 when
// K is a multiple of 4, else 2 when K is even, else K). A unit of four rows
// is the shape where every wave owns one row. 16 rows in one unit left each
// wave four rows and each workgroup a single 256-token tile (8 x 16 rows at
// ~9k tokens: 29.5 us; units of eight rows 34.4 us; of four 25.4 us, for
// four times the key reads).
static int rows_group(int K) { return K % 4 == 0 ? 4 : K % 2 == 0 ? 2 : K; }

template <int D, bool ONE_ROW, bool GM, int TILE = kIdxTile>
static void launch_one(const LaunchShape &ls, dim3 grid, const uint16_t *q_idx, const float *w,
                       const uint16_t *k_normed, const int32_t *seq_lens, float *scores,
                       uint32_t *gm4, uint32_t *gm32, hipStream_t stream, KTimer t)
{
    hipExtLaunchKernelGGL((k_index_scores<D, ONE_ROW, GM, TILE>), grid, dim3(kIdxThreads), 0, stream,
                          t.start, t.stop, 0u,
                       q_idx, w, k_normed, seq_lens, scores, gm4, gm32, ls.num_seqs,
                       ls.rows_per_seq, rows_group(ls.rows_per_seq),
                       ls.index_heads, (int64_t)ls.k_capacity, ls.max_len, score_stride(ls));
}

// Tokens per tile of the K-row pass, by rows per unit. With two or four
// rows every wave owns whole rows, and 128-token tiles give each workgroup
// twice as many steps of its load/compute pipeline (four instead of two at
// the 16 x 4 verify shape: 25.7 -> 23.3 us measured); the first tile's wait
// and the last tile's compute, which nothing overlaps, are then half as
// long. The pair walk needs an even item count per wave, so an odd unit
// keeps 256.
static int rows_tile(int KG) { return KG == 2 || KG == 4 ? 128 : kIdxTile; }
// Tokens per tile of the single-row pass. When even rows of max_len tokens
// would give each workgroup at most one 256-token tile, 128-token tiles
// double the workgroups that share the row and halve each one's serial
// load-then-compute (1 x 8192: 6.2 -> 5.4 us measured); with more tiles than
// workgroups, 256 is faster (8 x 131072: 45.9 against 49.5 us).
static int row_tile(const LaunchShape &ls)
{
    return (int64_t)ls.num_seqs * ((ls.max_len + kIdxTile - 1) / kIdxTile) <= kIdxWgTarget ? 128 : kIdxTile;
}

template <int D>
static void launch_d(const LaunchShape &ls, dim3 grid, const uint16_t *q_idx, const float *w,
                     const uint16_t *k_normed, const int32_t *seq_lens, float *scores,
                     uint32_t *gm4, uint32_t *gm32, hipStream_t stream, KTimer t)
{
    const bool one = ls.rows_per_seq == 1;
    const bool gm = gm4 != nullptr;
    const bool half = one ? row_tile(ls) == 128 : rows_tile(rows_group(ls.rows_per_seq)) == 128;
    if (one && gm && half)
        launch_one<D, true, true, 128>(ls, grid, q_idx, w, k_normed, seq_lens, scores, gm4, gm32,
                                       stream, t);
    else if (one && half)
        launch_one<D, true, false, 128>(ls, grid, q_idx, w, k_normed, seq_lens, scores, gm4, gm32,
                                        stream, t);
    else if (one && gm)
        launch_one<D, true, true>(ls, grid, q_idx, w, k_normed, seq_lens, scores, gm4, gm32,
                                  stream, t);
    else if (one)
        launch_one<D, true, false>(ls, grid, q_idx, w, k_normed, seq_lens, scores, gm4, gm32,
                                   stream, t);
    else if (gm && half)
        launch_one<D, false, true, 128>(ls, grid, q_idx, w, k_normed, seq_lens, scores, gm4, gm32,
                                        stream, t);
    else if (half)
        launch_one<D, false, false, 128>(ls, grid, q_idx, w, k_normed, seq_lens, scores, gm4,
                                         gm32, stream, t);
    else if (gm)
        launch_one<D, false, true>(ls, grid, q_idx, w, k_normed, seq_lens, scores, gm4, gm32,
                                   stream, t);
    else
        launch_one<D, false, false>(ls, grid, q_idx, w, k_normed, seq_lens, scores, gm4, gm32,
                                    stream, t);
}

int launch_index_scores(const LaunchShape &ls, const uint16_t *q_idx, const float *w,
                        const uint16_t *k_normed, const int32_t *seq_lens, float *scores,
                        uint32_t *gm4, uint32_t *gm32, hipStream_t stream, KTimer t)
{
    if ((gm4 == nullptr) != (gm32 == nullptr))
        return -1;
    // About kIdxWgTarget workgroups in all, balanced over the sequences by
    // their device-side lengths; each walks every W-th tile of one sequence
    // with the next tile's loads in flight.
    // enough for any split of the tiles over the units
    dim3 grid(kIdxWgTarget + ls.num_seqs * (ls.rows_per_seq / rows_group(ls.rows_per_seq)));
    if (ls.index_dim == 128)
        launch_d<128>(ls, grid, q_idx, w, k_normed, seq_lens, scores, gm4, gm32, stream, t);
    else if (ls.index_dim == 64)
        launch_d<64>(ls, grid, q_idx, w, k_normed, seq_lens, scores, gm4, gm32, stream, t);
    else
        return -1;
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

} // namespace dsa
