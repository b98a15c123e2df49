// mla_decode.hip -- FP8 paged NoPE MLA gather-attend on the gfx950 matrix cores.
//
// For each row r and head h, over the n_r = min(top_k, L_r) selected tokens
// (glm5next_dsa/layer.rs source page: module header, fourth trap; doc of
// `attend_rows`; the `kv_scale` field; `decode_k` for the paged slot):
//   c_j = kv_scale * e4m3(latent row of token sel[r, j])
//   z_j = sm_scale * q[r, h, :] . c_j,   out[r, h, :] = sum_j softmax(z)_j c_j
//
// Decomposition (a function of the row alone, never of R, so every row is
// bit-reproducible whichever rows share a launch):
//  - A row's selection is cut into chunks of kAttChunk (256) slots, eight
//    steps of 32 tokens. One workgroup of 8 waves covers one chunk for a
//    group of G heads (16, 32 or 64), in four phases, every wave in each:
//  1. Gather: wave w resolves step w's 32 slots through the block table and
//     copies their FP8 latent rows (512 bytes each) from HBM straight into
//     its LDS step tile with the gfx950 LDS-direct loads
//     (global_load_lds_dwordx4: 16 bytes per lane, no registers). Rows are
//     token-major in a tile, their 16-byte chunks XOR-swizzled by the row
//     index, so the operand reads below touch every LDS bank evenly. One
//     barrier publishes all eight tiles.
//  2. QK: S^T[token, head] = tile (16 tokens x latent) x q^T on 16x16x32
//     bf16 MFMA, one chain of 16 k-steps per (16-token tile, 16-head tile);
//     the FP8 operand is converted to bf16 in registers (exact: every E4M3
//     value is a bf16 value; kv_scale is folded into the logit scale and the
//     output). Each wave owns one head tile and 2, 4 or 8 of the 16 token
//     tiles; the per-head maxima of the chunk meet through LDS.
//  3. Softmax over the chunk, in fp32 and exact: m the chunk's largest
//     logit (log2 domain), p = exp2(z - m) rounded to bf16 for PV, and
//     l = the 16 token-tile sums added in tile order (each tile sum in a
//     fixed lane order). P goes to LDS in the PV operand's k order, 32 heads
//     at a time. exp2 is the hardware exponential: for z - m >= -126 the
//     same bits as the library's exp2f, which wraps it in a rescaling for
//     subnormal results (five more instructions per value); below that p
//     is flushed to zero, where exp2f gives a subnormal far under what the
//     bf16 output resolves. A step whose every slot holds a selected token
//     skips the mask.
//  4. PV, transposed: O^T[latent col, head] += V^T P^T, the tile as A through
//     the gfx950 8-bit transpose reads (ds_read_b64_tr_b8: a 16-lane group
//     receives 8 token rows of one 16-column block) converted to bf16, P as
//     B; wave w holds latent columns 64 w .. 64 w + 63 of every head, one
//     MFMA chain over the eight steps per (16-column tile, 16-head tile).
//  Every sum above has one order whatever G, so a head's output is the same
//  bits whichever heads share its workgroup.
//  - A row with one chunk writes its bf16 output directly. Otherwise every
//    chunk writes (m, l) in fp32 and its unnormalised O rounded to bf16 (the
//    precision of the output; half the partial traffic), and k_mla_merge
//    folds them in chunk order 0, 1, 2, ... with the same fp32 formula for
//    every row.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kAttThreads = 512;  // 8 waves, two per SIMD
constexpr int kAttWaves = kAttThreads / kWave;
constexpr int kStep = 32;         // tokens per step tile
constexpr int kLat = 512;         // latent width (bytes of an FP8 row)
constexpr int kMaxSteps = kAttChunk / kStep;     // 8 (one per wave)
constexpr int kTokTiles = kAttChunk / 16;        // 16-token MFMA tiles of a chunk
constexpr int kTileBytes = kStep * kLat;         // 16 KiB of FP8 per step
constexpr int kDmaPerStep = kTileBytes / (kWave * 16); // LDS-direct loads per step tile (16)
constexpr int kPvColTiles = kLat / 16 / kAttWaves;     // 16-column tiles per wave (4)
// P in LDS: every head of the group for as many tokens as fit beside the
// ring (256 with 16 or 32 heads, 128 with 64: then PV runs in two passes
// over the chunk's halves). P rows are padded by 16 bytes: 16 consecutive
// heads read at one 16-byte column hit 16 distinct 4-bank groups.
template <int G> constexpr int p_tokens() { return G == 64 ? kAttChunk / 2 : kAttChunk; }
template <int G> constexpr int p_row_bytes() { return 2 * p_tokens<G>() + 16; }
constexpr float kNegInf = -__builtin_huge_valf();
static_assert(kMaxSteps == kAttWaves, "wave w gathers step w");

typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) void lds_void;

// Byte offset, inside a step tile, of 16-byte chunk `chunk` (0..31) of token
// row `row` (0..31): rows are 512 bytes apart and their chunks XOR-swizzled
// by the row index.
__device__ __forceinline__ int tile_off(int row, int chunk) { return row * kLat + ((chunk ^ row) << 4); }

// Eight E4M3 bytes (two dwords) -> eight bf16, exact, in byte order.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(v2i w)
{
    u32x4 r;
    r.x = e4m3x2_to_bf16x2_exact<false>((uint32_t)w.x);
    r.y = e4m3x2_to_bf16x2_exact<true>((uint32_t)w.x);
    r.z = e4m3x2_to_bf16x2_exact<false>((uint32_t)w.y);
    r.w = e4m3x2_to_bf16x2_exact<true>((uint32_t)w.y);
    return as_bf16x8(r);
}

// Folding the per-chunk partials of one (row, head) at latent columns
// d .. d + 7, strictly in chunk order 0, 1, 2, ... with one fp32 formula.
// Partials are loaded in unrolled batches (independent loads in flight), then
// folded; straight-line code with selects, so the batch stays in registers. A
// batch is the chunk count of a row at top_k = 2048 (8 x 256 slots): a larger
// one re-reads the last chunk (measured: 16 cost 3.5 us per step at
// 64 x 16.4k).
constexpr int kFoldBatch = 8;
constexpr int kFoldCols = 8; // latent columns per lane (16 bytes of bf16)
struct FoldState {
    float m, l;
    float acc[kFoldCols];
};
struct FoldBatch {
    float2 ml[kFoldBatch];
    u32x4 ov[kFoldBatch];
};
// chunks past `last` re-read it (branch-free; they are not folded)
__device__ __forceinline__ void fold_load(const uint16_t *part_o, const float2 *part_ml, int64_t pbase,
                                          int G, int c0, int last, int d, FoldBatch &b)
{
#pragma unroll
    for (int k = 0; k < kFoldBatch; k++) {
        const int64_t pi = pbase + (int64_t)min(c0 + k, last) * G;
        b.ml[k] = part_ml[pi];
        b.ov[k] = *(const u32x4 *)(part_o + pi * kLat + d);
    }
}
__device__ __forceinline__ void fold_step(int c0, int nch, const FoldBatch &b, FoldState &f)
{
#pragma unroll
    for (int k = 0; k < kFoldBatch; k++) {
        const float m_new = __builtin_fmaxf(f.m, b.ml[k].x);
        // a chunk past the last, or one with nothing selected so far, leaves
        // the state untouched
        const bool use = (c0 + k < nch) && (m_new != kNegInf);
        const float a = use ? exp2f(f.m - m_new) : 1.0f;
        const float e = use ? exp2f(b.ml[k].x - m_new) : 0.0f;
        f.l = use ? __builtin_fmaf(b.ml[k].y, e, f.l * a) : f.l;
#pragma unroll
        for (int i = 0; i < kFoldCols; i++) {
            const uint32_t w = b.ov[k][i / 2];
            const float o = __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
            f.acc[i] = use ? __builtin_fmaf(o, e, f.acc[i] * a) : f.acc[i];
        }
        f.m = use ? m_new : f.m;
    }
}
__device__ __forceinline__ u32x4 fold_output(const FoldState &f, float kv_scale)
{
    const float inv = f.l > 0.0f ? kv_scale / f.l : 0.0f;
    u32x4 packed;
#pragma unroll
    for (int i = 0; i < 4; i++)
        packed[i] = pack_bf16x2(f.acc[2 * i] * inv, f.acc[2 * i + 1] * inv);
    return packed;
}

// The 4 x 4 transpose of 16-lane rows and four registers: on return, row g
// of r[j] holds what row j of r[g] held (gfx950 lane swaps: the 32-lane swap
// exchanges rows 2-3 of its first operand with rows 0-1 of its second, the
// 16-lane swap rows 1 and 3 of its first with rows 0 and 2 of its second).
__device__ __forceinline__ void transpose_rows(uint32_t (&r)[4])
{
    auto s02 = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);
    auto s13 = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
    auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
    auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
    r[0] = s01[0];
    r[1] = s01[1];
    r[2] = s23[0];
    r[3] = s23[1];
}

// G: heads per workgroup (16, 32 or 64); it changes where the work runs,
// never a result.
template <int G>
__global__ __launch_bounds__(kAttThreads, 1) void k_mla_decode(
    const uint16_t *__restrict__ q, const uint8_t *__restrict__ kv,
    const int32_t *__restrict__ bt, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ sel, uint16_t *__restrict__ part_o, float2 *__restrict__ part_ml,
    uint16_t *__restrict__ out, int K, int H, int top_k, int ps, int max_blocks, int num_pages,
    int max_len, float kv_scale, float qk_log2, int nch_max, int hg_count)
{
    constexpr int kHt = G / 16;                 // 16-head tiles of the group
    constexpr int kWavesPerHt = kAttWaves / kHt; // QK: waves sharing one head tile (8, 4, 2)
    constexpr int kTpw = kTokTiles / kWavesPerHt; // QK: token tiles of one wave (2, 4, 8)
    constexpr int kPTok = p_tokens<G>();         // tokens whose P is in LDS at once
    constexpr int kPRowBytes = p_row_bytes<G>();
    constexpr int kPasses = kAttChunk / kPTok;   // PV passes over the chunk (1, 1, 2)
    constexpr int kStepsPerPass = kPTok / kStep;
    static_assert(kHt == 1 || kHt == 2 || kHt == 4, "16, 32 or 64 heads");
    __shared__ __align__(16) uint8_t ring[kMaxSteps * kTileBytes]; // FP8 step tiles (128 KiB)
    // bf16 P of one pass; with 16 heads it first holds the group's query
    // (16 heads x 1 KiB, loaded once instead of once per wave)
    constexpr int kQLds = kHt == 1;
    constexpr int kPBytes = G * kPRowBytes;
    __shared__ __align__(16) uint8_t pbuf[kQLds && 16 * 2 * kLat > kPBytes ? 16 * 2 * kLat : kPBytes];
    __shared__ float wmax[kAttWaves][16];       // per-wave maxima of its head tile's heads
    __shared__ float tsum[kTokTiles][G];        // per-token-tile sums of p
    __shared__ __align__(16) uint8_t vmask[kAttChunk]; // slot holds a selected token
    __shared__ uint8_t vfull[kMaxSteps];                // every slot of step s does

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int g = lane >> 4;
    const int n16 = lane & 15;
    const int r = blockIdx.y;
    const int c = blockIdx.x % nch_max;
    const int hg = blockIdx.x / nch_max;
    const int s = r / K;
    const int slot0 = c * kAttChunk;
    // The row length and this lane's selected id are requested together
    // (the id's index is in bounds whatever the length: chunk c exists for
    // top_k, and past the row's n the id is loaded but not used); the
    // block-table lookup follows, and only then the query, so that neither
    // resolution load waits behind the query's in the in-order return queue.
    const int slot = kStep * wave + (lane & 31); // wave w resolves step w (both half-waves)
    // QK ownership. A lane past the group's last head scores with head H-1's
    // query: its results are never stored, and a head's arithmetic never
    // involves another head's.
    const int ht = wave / kWavesPerHt;           // head tile of this wave's QK
    const int tt0 = (wave % kWavesPerHt) * kTpw; // its first token tile
    const int hl = ht * 16 + n16;                // this lane's head within the group
    if constexpr (kQLds) {
        // 16 heads: wave w copies heads 2 w and 2 w + 1 (1 KiB each) into LDS
        // first (no dependence on anything); the 16-byte chunk c of head h
        // sits in slot c ^ (h & 15), so the 16 heads read at one column hit
        // 16 distinct bank groups (lane j fetches the chunk its slot j holds)
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int hq = 2 * wave + i;
            const uint8_t *gsrc = (const uint8_t *)(q + ((int64_t)r * H + min(hg * G + hq, H - 1)) * kLat) +
                                  16 * (lane ^ (hq & 15));
            __builtin_amdgcn_global_load_lds((const void *)gsrc, (lds_void *)(pbuf + hq * 2 * kLat), 16,
                                             0, 0);
        }
    }
    const int t_sel = sel[(int64_t)r * top_k + min(slot0 + slot, top_k - 1)];
    const int L = min(max(seq_lens[r], 0), max_len);
    const int n = min(top_k, L);
    const int nch = (n + kAttChunk - 1) / kAttChunk;
    const int h0 = hg * G;         // first head of the group
    const int nh = min(G, H - h0); // heads of the group that exist

    if (n == 0) {
        if (c == 0) {
            for (int i = tid; i < G * kLat; i += kAttThreads) {
                const int h = h0 + i / kLat;
                if (h < H)
                    out[((int64_t)r * H + h) * kLat + (i % kLat)] = 0;
            }
        }
        return;
    }
    if (c >= nch)
        return;
    const int nslots = min(n - slot0, kAttChunk);

    // ================= phase 1: resolve and gather step `wave` =================
    int row = -1;
    if (slot < nslots && t_sel >= 0 && t_sel < L) {
        const int page = bt[(int64_t)s * max_blocks + t_sel / ps];
        if (page >= 0 && page < num_pages)
            row = page * ps + t_sel % ps;
    }

    // 32 or 64 heads: the query goes to registers, requested after the
    // block-table lookup so that neither resolution load waits behind it
    // (measured: requesting it after the tile copies instead is slower)
    u32x4 qr[16]; // head hl, latent dims 32 ks + 8 g .. +7 (the B operand)
    if constexpr (!kQLds) {
        const uint16_t *qrow = q + ((int64_t)r * H + min(h0 + hl, H - 1)) * kLat + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 16; ks++)
            qr[ks] = *(const u32x4 *)(qrow + 32 * ks);
    }

    if (lane < 32)
        vmask[slot] = row >= 0 ? 1 : 0;
    if (lane == 0)
        vfull[wave] = (__ballot(row >= 0) & 0xFFFFFFFFull) == 0xFFFFFFFFull ? 1 : 0;
    {
        uint8_t *tile = ring + wave * kTileBytes;
        // A skipped slot (past the chunk, or out of contract) copies one of
        // the step's selected rows instead: finite data that its zero
        // probability removes exactly, and never a read of the skipped
        // token. A step with no selected row is zeroed.
        const uint64_t any = __ballot(row >= 0) & 0xFFFFFFFFull;
        if (any != 0) {
            const int sub = __builtin_amdgcn_readlane(row, __ffsll((unsigned long long)any) - 1);
            const int src = row >= 0 ? row : sub;
            const int half = lane >> 5;
            // load i: tile rows 2 i (lanes 0-31) and 2 i + 1 (lanes 32-63);
            // lane j fetches the global chunk that lands in slot j & 31 of
            // its row (the swizzle's inverse)
#pragma unroll
            for (int i = 0; i < kDmaPerStep; i++) {
                const int rowa = __builtin_amdgcn_readlane(src, 2 * i);
                const int rowb = __builtin_amdgcn_readlane(src, 2 * i + 1);
                const int trow = 2 * i + half;
                const int grow = half ? rowb : rowa;
                const uint8_t *gsrc = kv + (int64_t)grow * kLat + 16 * ((lane & 31) ^ trow);
                __builtin_amdgcn_global_load_lds((const void *)gsrc, (lds_void *)(tile + 2 * i * kLat),
                                                 16, 0, 0);
            }
        } else {
            for (int i = lane; i < kTileBytes / 16; i += kWave)
                *(u32x4 *)(tile + 16 * i) = u32x4{0u, 0u, 0u, 0u};
        }
    }
    if constexpr (kQLds) {
        // The query copies were issued before the resolution loads, and
        // every wave drained those (in order) before its tile copies went
        // out, so after a plain barrier every head's query is in LDS; the
        // barrier does not wait for the tile copies, which stay in flight
        // while the query goes to registers.
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int ks = 0; ks < 16; ks++)
            qr[ks] = *(const u32x4 *)(pbuf + n16 * 2 * kLat + 16 * ((4 * ks + g) ^ n16));
        // a wave's two token tiles are its own step: its loads landing is
        // enough (P overwrites the query area only after the maxima barrier,
        // which every wave reaches after its QK has consumed the query)
        __builtin_amdgcn_s_waitcnt(0xc07f & ~(0x3 << 14) & ~0xF); // vmcnt(0)
    } else {
        __syncthreads(); // every tile landed (each wave drained its own loads), masks set
    }

    // ================= phase 2: QK and the chunk's maxima =================
    // lane: head hl, tokens 16 tt + 4 g + v of each of its token tiles
    floatx4 z[kTpw];
    // The FP8 operands of four k-steps of a tile pair (tiles tt, tt + 1, the
    // two halves of step tt / 2); the next group's are requested before this
    // group's conversions and products, so the LDS reads stay in flight
    // behind them.
    auto qk_operands = [&](int j, int k0, v2i (&a)[2][4]) {
        const uint8_t *tb = ring + ((tt0 + j) >> 1) * kTileBytes;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int chunk = 2 * (k0 + k) + (g >> 1);
#pragma unroll
            for (int h = 0; h < 2; h++)
                a[h][k] = *(const v2i *)(tb + tile_off(16 * h + n16, chunk) + 8 * (g & 1));
        }
    };
    // (with 64 heads the registers this takes cost more than it saves:
    // measured, so that form requests each group's operands in turn)
    constexpr bool kPf = kHt < 4;
    v2i a[2][4];
    if (kPf)
        qk_operands(0, 0, a);
#pragma unroll
    for (int j = 0; j < kTpw; j += 2) {
        floatx4 acc[2] = {floatx4{0.0f, 0.0f, 0.0f, 0.0f}, floatx4{0.0f, 0.0f, 0.0f, 0.0f}};
        const int tt = tt0 + j; // even: tiles tt, tt + 1 are the two halves of step tt / 2
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
            if (!kPf)
                qk_operands(j, k0, a);
            v2i an[2][4];
            const int nj = k0 == 12 ? j + 2 : j;
            if (kPf && nj < kTpw)
                qk_operands(nj, k0 == 12 ? 0 : k0 + 4, an);
#pragma unroll
            for (int k = 0; k < 4; k++) {
#pragma unroll
                for (int h = 0; h < 2; h++)
                    acc[h] = mfma16x16x32(fp8x8_to_bf16x8(a[h][k]), as_bf16x8(qr[k0 + k]), acc[h]);
            }
            if (kPf && nj < kTpw) {
#pragma unroll
                for (int k = 0; k < 4; k++)
#pragma unroll
                    for (int h = 0; h < 2; h++)
                        a[h][k] = an[h][k];
            }
        }
        // a step whose every slot holds a selected token needs no mask
        if (__builtin_amdgcn_readfirstlane(vfull[tt >> 1])) {
#pragma unroll
            for (int h = 0; h < 2; h++)
#pragma unroll
                for (int v = 0; v < 4; v++)
                    z[j + h][v] = acc[h][v] * qk_log2;
        } else {
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const uint32_t mw = *(const uint32_t *)(vmask + 16 * (tt + h) + 4 * g);
#pragma unroll
                for (int v = 0; v < 4; v++)
                    z[j + h][v] = ((mw >> (8 * v)) & 0xFFu) ? acc[h][v] * qk_log2 : kNegInf;
            }
        }
    }
    {
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < kTpw; j++)
#pragma unroll
            for (int v = 0; v < 4; v++)
                mx = __builtin_fmaxf(mx, z[j][v]);
        mx = max_xor32(max_xor16(mx));
        if (g == 0)
            wmax[wave][n16] = mx;
    }
    __syncthreads(); // wave maxima

    // ================= phase 3: softmax over the chunk =================
    float m = kNegInf; // the chunk's largest logit of head hl (exact: order-free)
#pragma unroll
    for (int w = 0; w < kWavesPerHt; w++)
        m = __builtin_fmaxf(m, wmax[ht * kWavesPerHt + w][n16]);
    const float m_use = (m == kNegInf) ? 0.0f : m;
    u32x4 pk[kTpw / 2]; // bf16 P of each of this wave's steps, PV k order
#pragma unroll
    for (int j = 0; j < kTpw; j += 2) {
        float p[8];
#pragma unroll
        for (int h = 0; h < 2; h++) {
#pragma unroll
            for (int v = 0; v < 4; v++)
                p[4 * h + v] = __builtin_amdgcn_exp2f(z[j + h][v] - m_use);
            // tile sum: this lane's four tokens, then the four lane groups,
            // in one fixed order (the swaps add commuted pairs: same bits)
            float ts = (p[4 * h] + p[4 * h + 1]) + (p[4 * h + 2] + p[4 * h + 3]);
            ts = add_xor32(add_xor16(ts));
            if (g == 0)
                tsum[tt0 + j + h][hl] = ts;
        }
        pk[j / 2].x = pack_bf16x2(p[0], p[1]);
        pk[j / 2].y = pack_bf16x2(p[2], p[3]);
        pk[j / 2].z = pack_bf16x2(p[4], p[5]);
        pk[j / 2].w = pack_bf16x2(p[6], p[7]);
    }

    // ================= phase 4: PV =================
    // The tile as A through 8-bit transpose reads: in lane group g, lane
    // pair k supplies token row 4 g + k (k < 4) or 16 + 4 g + k - 4, so lane
    // n16 receives column 16 (4 wave + i) + n16 of those 8 rows (k-slot j <->
    // token 16 (j >> 2) + 4 g + (j & 3) of the step, the order P is written
    // in); P as B. A lane ends with 4 consecutive columns of one head.
    const int kp = n16 >> 1;
    const int trrow = (kp < 4) ? 4 * g + kp : 16 + 4 * g + (kp - 4);
    floatx4 o[kHt][kPvColTiles]; // O^T[cols 64 wave + 16 i + 4 g + e][head 16 mt + n16]
    float lh[kHt];               // l of head 16 mt + n16
#pragma unroll
    for (int mt = 0; mt < kHt; mt++)
#pragma unroll
        for (int i = 0; i < kPvColTiles; i++)
            o[mt][i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int pass = 0; pass < kPasses; pass++) {
        if (pass > 0)
            __syncthreads(); // the previous pass's P reads are done
        // this wave's P of the pass's steps
#pragma unroll
        for (int j = 0; j < kTpw; j += 2) {
            const int st = (tt0 + j) >> 1;
            if (st / kStepsPerPass == pass)
                *(u32x4 *)(pbuf + hl * kPRowBytes + 2 * (kStep * (st % kStepsPerPass) + 8 * g)) = pk[j / 2];
        }
        __syncthreads(); // P of the pass (and, at the first, every tile sum)
        if (pass == 0) {
            // l of each head: the token-tile sums in tile order
#pragma unroll
            for (int mt = 0; mt < kHt; mt++) {
                float acc = 0.0f;
#pragma unroll
                for (int tt = 0; tt < kTokTiles; tt++)
                    acc += tsum[tt][16 * mt + n16];
                lh[mt] = acc;
            }
            if (nch > 1 && wave % kWavesPerHt == 0 && g == 0 && hl < nh) {
                const int64_t pb = (((int64_t)r * hg_count + hg) * nch_max + c) * G;
                part_ml[pb + hl] = float2{m, lh[ht]};
            }
        }
#pragma unroll
        for (int sp = 0; sp < kStepsPerPass; sp++) {
            const int st = pass * kStepsPerPass + sp;
            const uint8_t *tb = ring + st * kTileBytes;
            v2i raw[kPvColTiles];
#pragma unroll
            for (int i = 0; i < kPvColTiles; i++)
                raw[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (lds_v2i *)(tb + tile_off(trrow, kPvColTiles * wave + i) + 8 * (n16 & 1)));
            bf16x8 pa[kHt];
#pragma unroll
            for (int mt = 0; mt < kHt; mt++)
                pa[mt] = as_bf16x8(*(const u32x4 *)(pbuf + (mt * 16 + n16) * kPRowBytes +
                                                    2 * (kStep * sp + 8 * g)));
#pragma unroll
            for (int i = 0; i < kPvColTiles; i++) {
                const bf16x8 va = fp8x8_to_bf16x8(raw[i]);
#pragma unroll
                for (int mt = 0; mt < kHt; mt++) // head tiles past the group's heads see P = 0
                    o[mt][i] = mfma16x16x32(va, pa[mt], o[mt][i]);
            }
        }
    }

    if constexpr (kHt < 4) {
        // Output straight from registers as whole 128-byte lines: row g of
        // column tile i holds columns 16 (4 w + i) + 4 g .. + 3 of head
        // 16 mt + n16; after the 4 x 4 transpose of the lane rows, row g holds
        // the 16 columns 16 (4 w + g) .. + 15 (8-byte stores of the untransposed
        // layout leave lines partly written, and the kernel's end waits for
        // their write-back; parking O in LDS to write whole rows costs a barrier
        // and the copies through LDS)
        const int64_t pbase = (((int64_t)r * hg_count + hg) * nch_max + c) * G;
#pragma unroll
        for (int mt = 0; mt < kHt; mt++) {
            const float sc = (nch == 1) ? (lh[mt] > 0.0f ? kv_scale / lh[mt] : 0.0f) : 1.0f;
            uint32_t lo4[kPvColTiles], hi4[kPvColTiles];
#pragma unroll
            for (int i = 0; i < kPvColTiles; i++) {
                lo4[i] = pack_bf16x2(o[mt][i][0] * sc, o[mt][i][1] * sc);
                hi4[i] = pack_bf16x2(o[mt][i][2] * sc, o[mt][i][3] * sc);
            }
            transpose_rows(lo4);
            transpose_rows(hi4);
            const int hrow = 16 * mt + n16;
            const int col = 16 * (kPvColTiles * wave + g);
            if (hrow < nh) {
                const u32x4 v0 = u32x4{lo4[0], hi4[0], lo4[1], hi4[1]};
                const u32x4 v1 = u32x4{lo4[2], hi4[2], lo4[3], hi4[3]};
                if (nch == 1) {
                    uint16_t *orow = out + ((int64_t)r * H + h0 + hrow) * kLat + col;
                    *(u32x4 *)orow = v0;
                    *(u32x4 *)(orow + 8) = v1;
                } else {
                    // streaming stores for partials: read once, by the merge
                    uint16_t *orow = part_o + (pbase + hrow) * kLat + col;
                    __builtin_nontemporal_store(v0, (u32x4 *)orow);
                    __builtin_nontemporal_store(v1, (u32x4 *)(orow + 8));
                }
            }
        }
    } else {
        // 64 heads (four head tiles a wave): parking O in the idle ring and
        // writing whole 1 KiB head rows measured faster than the direct
        // stores above (batched: 23.2 against 23.8 us)
        __syncthreads(); // every wave is done with the ring

        // Output through LDS: the waves park O (G heads x 512 columns, bf16) in
        // the idle ring, then write it back as whole 1 KiB head rows with 16-byte
        // stores (measured faster than 8-byte stores straight from registers,
        // with 16 heads as with 64).
        constexpr int kORowBytes = 2 * kLat + 16; // padded: 16 rows at one column spread over the banks
        static_assert(G * kORowBytes <= (int)sizeof(ring), "O fits the ring");
#pragma unroll
        for (int mt = 0; mt < kHt; mt++) {
            const float sc = (nch == 1) ? (lh[mt] > 0.0f ? kv_scale / lh[mt] : 0.0f) : 1.0f;
#pragma unroll
            for (int i = 0; i < kPvColTiles; i++) {
                u32x2 pw;
                pw.x = pack_bf16x2(o[mt][i][0] * sc, o[mt][i][1] * sc);
                pw.y = pack_bf16x2(o[mt][i][2] * sc, o[mt][i][3] * sc);
                *(u32x2 *)(ring + (16 * mt + n16) * kORowBytes + 2 * (16 * (kPvColTiles * wave + i) + 4 * g)) = pw;
            }
        }
        __syncthreads();
        const int64_t pbase = (((int64_t)r * hg_count + hg) * nch_max + c) * G;
#pragma unroll
        for (int it = 0; it < G * (kLat * 2 / 16) / kAttThreads; it++) {
            const int e = it * kAttThreads + tid; // 16-byte piece e of the G x 1 KiB block
            const int hrow = e / (kLat * 2 / 16);
            const int cb = 16 * (e % (kLat * 2 / 16));
            if (hrow < nh) {
                const u32x4 val = *(const u32x4 *)(ring + hrow * kORowBytes + cb);
                uint16_t *orow = (nch == 1) ? out + ((int64_t)r * H + h0 + hrow) * kLat
                                            : part_o + (pbase + hrow) * kLat;
                // streaming store for partials: read once, by the merge
                if (nch == 1)
                    *(u32x4 *)((uint8_t *)orow + cb) = val;
                else
                    __builtin_nontemporal_store(val, (u32x4 *)((uint8_t *)orow + cb));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// More (row, chunk) units of 64 heads than CUs: one workgroup per CU takes a
// run of consecutive units in turn (chunks of one row, mostly: the query
// stays in registers), so that the ring never idles between units. While
// unit u runs its softmax and P.V, the next unit's length and selected ids
// are requested, and its tile copies go out as P.V frees the ring (steps 0-3
// after the first P.V pass, 4-7 after the second); unit u's output is stored
// during the next unit's QK. QK ownership: wave w scores token tile
// 2 st + (w & 1) of every step st for head tile w >> 1 (two waves a head
// tile, as in k_mla_decode<64>). Every element's arithmetic is k_mla_decode's
// (the same MFMA chains, maxima, exponentials, tile sums, P rounding and P.V
// step order), so a row's output has the same bits from either kernel.
//
// The pointers carry no __restrict__: loads through const restrict pointers
// count as invariant, and the next unit's query and id loads must stay where
// they are issued rather than sink to their use.
constexpr int kWaitVmLgkm0 = 0x0070; // s_waitcnt vmcnt(0) lgkmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;   // s_waitcnt lgkmcnt(0)

// The thread id through an opaque move: lane-derived addresses computed from
// it stay inside the unit loop instead of being hoisted out of it (with every
// LDS and global address of a unit held in registers, the kernel spills).
__device__ __forceinline__ int opaque_tid()
{
    int t;
    __asm__ volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
    return t;
}


// A workgroup barrier that publishes this wave's LDS writes but does not wait
// for its vector-memory operations (tile copies stay in flight across it).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

__global__ __launch_bounds__(kAttThreads, 1) void k_mla_decode_pipe(
    const uint16_t *q, const uint8_t *kv, const int32_t *bt, const int32_t *seq_lens,
    const int32_t *sel, uint16_t *part_o, float2 *part_ml, uint16_t *out, int K, int H, int top_k,
    int ps, int max_blocks, int num_pages, int max_len, float kv_scale, float qk_log2, int nch_max,
    int hg_count, int units)
{
    constexpr int G = kAttHeads;
    constexpr int kHt = G / 16;                  // 4 head tiles
    constexpr int kPTok = p_tokens<G>();         // P of 128 tokens in LDS at once
    constexpr int kPRowBytes = p_row_bytes<G>();
    constexpr int kStepsPerPass = kPTok / kStep; // 4
    static_assert(kAttWaves == 2 * kHt && kMaxSteps == 8 && kStepsPerPass == 4,
                  "two waves a head tile; eight steps, P.V in two passes of four");
    __shared__ __align__(16) uint8_t ring[kMaxSteps * kTileBytes]; // FP8 step tiles (128 KiB)
    __shared__ __align__(16) uint8_t pbuf[G * kPRowBytes];        // bf16 P of one pass
    __shared__ float wmax[kAttWaves][16];
    __shared__ float tsum[kTokTiles][G];
    __shared__ __align__(16) uint8_t vmask[kAttChunk];
    __shared__ uint8_t vfull[kMaxSteps];

    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int ht = wave >> 1;  // QK head tile
    const int par = wave & 1;  // QK token tile 2 st + par of step st
    const int per_row = hg_count * nch_max;
    // this workgroup's units: [ubeg, uend)
    const int upw = (units + (int)gridDim.x - 1) / (int)gridDim.x;
    const int ubeg = (int)blockIdx.x * upw;
    const int uend = min(ubeg + upw, units);
    // lane-derived values, recomputed where they are used
#define PIPE_LANE                                                                              \
    const int tid = opaque_tid();                                                              \
    const int lane = tid % kWave;                                                              \
    const int g = lane >> 4;                                                                   \
    const int n16 = lane & 15;                                                                 \
    const int slot = kStep * wave + (lane & 31); /* wave w copies step w of every unit */      \
    const int hl = ht * 16 + n16;                /* this lane's QK head within the group */    \
    (void)g;                                                                                   \
    (void)slot;                                                                                \
    (void)hl;

    // ---- the unit being prepared (uniform but for the lane's id and page) ----
    int nu = units, nr = 0, nhg = 0, nc = 0, nlen = 0, nnch = 0;
    int t_seln = 0, pagen = -1;
    auto issue_len = [&](int u) { // length and this lane's selected id of unit u
        PIPE_LANE
        nu = u;
        nr = u / per_row;
        const int rem = u - nr * per_row;
        nhg = rem / nch_max;
        nc = rem - nhg * nch_max;
        nlen = seq_lens[nr];
        t_seln = sel[(int64_t)nr * top_k + min(nc * kAttChunk + slot, top_k - 1)];
    };
    auto issue_q = [&](u32x4(&qd)[16]) { // the prepared unit's query (head tile ht)
        PIPE_LANE
        const uint16_t *qrow = q + ((int64_t)nr * H + min(nhg * G + hl, H - 1)) * kLat + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 16; ks++)
            qd[ks] = *(const u32x4 *)(qrow + 32 * ks);
    };
    // Settles the unit issue_a requested: an empty one (a row with nothing
    // selected, or a chunk past the row's selection) is skipped, the first
    // chunk of an empty row writing zeros, and the next candidate requested
    // in its place. Returns whether a unit with work is prepared; its lane's
    // page lookup is then in flight.
    auto finish_b = [&]() -> bool {
        PIPE_LANE
        while (nu < units) {
            const int L = min(max(__builtin_amdgcn_readfirstlane(nlen), 0), max_len);
            const int n = min(top_k, L);
            const int nch = (n + kAttChunk - 1) / kAttChunk;
            if (n > 0 && nc < nch) {
                const int nslots = min(n - nc * kAttChunk, kAttChunk);
                nnch = nch;
                pagen = -1;
                if (slot < nslots && t_seln >= 0 && t_seln < L)
                    pagen = bt[(int64_t)(nr / K) * max_blocks + t_seln / ps];
                return true;
            }
            if (n == 0 && nc == 0) {
                const int h0 = nhg * G;
                for (int i = tid; i < G * kLat; i += kAttThreads) {
                    const int h = h0 + i / kLat;
                    if (h < H)
                        out[((int64_t)nr * H + h) * kLat + (i % kLat)] = 0;
                }
            }
            if (nu + 1 >= uend) {
                nu = units;
                break;
            }
            issue_len(nu + 1);
        }
        return false;
    };
    // Wave w's step of the prepared unit: masks, then the LDS-direct copies of
    // its FP8 rows into ring slot w (a skipped slot copies one of the step's
    // selected rows; a step with none is zeroed), as k_mla_decode does.
    auto issue_tile = [&]() {
        PIPE_LANE
        const int row = (pagen >= 0 && pagen < num_pages) ? pagen * ps + t_seln % ps : -1;
        if (lane < 32)
            vmask[slot] = row >= 0 ? 1 : 0;
        uint8_t *tile = ring + wave * kTileBytes;
        const uint64_t any = __ballot(row >= 0) & 0xFFFFFFFFull;
        if (lane == 0)
            vfull[wave] = any == 0xFFFFFFFFull ? 1 : 0;
        if (any != 0) {
            const int sub = __builtin_amdgcn_readlane(row, __ffsll((unsigned long long)any) - 1);
            const int src = row >= 0 ? row : sub;
            const int half = lane >> 5;
#pragma unroll
            for (int i = 0; i < kDmaPerStep; i++) {
                const int rowa = __builtin_amdgcn_readlane(src, 2 * i);
                const int rowb = __builtin_amdgcn_readlane(src, 2 * i + 1);
                const int trow = 2 * i + half;
                const int grow = half ? rowb : rowa;
                const uint8_t *gsrc = kv + (int64_t)grow * kLat + 16 * ((lane & 31) ^ trow);
                __builtin_amdgcn_global_load_lds((const void *)gsrc, (lds_void *)(tile + 2 * i * kLat),
                                                 16, 0, 0);
            }
        } else {
            for (int i = lane; i < kTileBytes / 16; i += kWave)
                *(u32x4 *)(tile + 16 * i) = u32x4{0u, 0u, 0u, 0u};
        }
    };

    // ---- the first unit ----
    if (ubeg >= uend)
        return;
    issue_len(ubeg);
    if (!finish_b())
        return; // uniform: nothing to do
    int cr = nr, chg = nhg, cc = nc, cnch = nnch, cu = nu;
    issue_tile();
    u32x4 qr[16];
    issue_q(qr);
    // (every load of the first unit retired here, so that no wait for the
    // query lands inside the unit loop)
    __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);

    // ---- the previous unit's output, stored after the next unit's QK ----
    // (its O already rounded to bf16 as it is stored: scaled by kv_scale / l
    // for a row of one chunk, unscaled as a chunk partial)
    bool have_prev = false;
    int pr = 0, phg = 0, pc = 0, pnch = 0;
    float pm = 0.0f, plh = 0.0f; // (m, l) of head hl
    u32x2 pw[kHt][kPvColTiles];
#pragma unroll
    for (int mt = 0; mt < kHt; mt++)
#pragma unroll
        for (int i = 0; i < kPvColTiles; i++)
            pw[mt][i] = u32x2{0u, 0u};
    auto store_prev = [&](int mt0, int mt1) { // head tiles mt0 .. mt1 - 1
        PIPE_LANE
        const int h0 = phg * G;
        const int nh = min(G, H - h0);
        const int64_t pb = (((int64_t)pr * hg_count + phg) * nch_max + pc) * G;
        if (mt0 == 0 && pnch > 1 && par == 0 && g == 0 && hl < nh)
            part_ml[pb + hl] = float2{pm, plh};
        // Row g of column tile i holds columns 16 (4 w + i) + 4 g .. + 3 of
        // head 16 mt + n16; after the transpose, row g holds the 16 columns
        // 16 (4 w + g) .. + 15 (in four 8-byte pieces), so that the four rows
        // fill whole 128-byte lines (8-byte pieces spread over lines leave
        // them partly written, and the kernel's end waits for their
        // write-back).
#pragma unroll
        for (int mt = 0; mt < kHt; mt++) {
            if (mt < mt0 || mt >= mt1)
                continue;
            uint32_t lo[4], hi[4];
#pragma unroll
            for (int i = 0; i < kPvColTiles; i++) {
                lo[i] = pw[mt][i].x;
                hi[i] = pw[mt][i].y;
            }
            transpose_rows(lo);
            transpose_rows(hi);
            const int hrow = 16 * mt + n16;
            const int col = 16 * (kPvColTiles * wave + g);
            if (hrow < nh) {
                const u32x4 v0 = u32x4{lo[0], hi[0], lo[1], hi[1]};
                const u32x4 v1 = u32x4{lo[2], hi[2], lo[3], hi[3]};
                if (pnch == 1) {
                    uint16_t *orow = out + ((int64_t)pr * H + h0 + hrow) * kLat + col;
                    *(u32x4 *)orow = v0;
                    *(u32x4 *)(orow + 8) = v1;
                } else {
                    uint16_t *orow = part_o + (pb + hrow) * kLat + col;
                    __builtin_nontemporal_store(v0, (u32x4 *)orow);
                    __builtin_nontemporal_store(v1, (u32x4 *)(orow + 8));
                }
            }
        }
    };

    for (;;) {
        // ================= QK over step pairs =================
        floatx4 z[kMaxSteps]; // z[st]: token tile 2 st + par, head hl
        // the lane's operand offset in a step tile for each of the 16
        // k-steps: the same in every step, so that the four pairs' reads take
        // it as their base and the steps' tile offsets as immediates
        int qoff[16];
        {
            PIPE_LANE
#pragma unroll
            for (int kk = 0; kk < 16; kk++)
                qoff[kk] = tile_off(16 * par + n16, 2 * kk + (g >> 1)) + 8 * (g & 1);
        }
#pragma unroll
        for (int p = 0; p < kMaxSteps / 2; p++) {
            PIPE_LANE
            if (p == 0) {
                // every wave's copies landed (each waits for its own step),
                // then one barrier: one per step pair costs more than scoring
                // the first pairs while the last land saves (measured)
                __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
                __asm__ volatile("" ::: "memory");
                __builtin_amdgcn_s_barrier();
                __asm__ volatile("" ::: "memory");
            }
            // the previous unit's output, head tile p in pair p: after the
            // copy wait (a store issued before it would hold that wait)
            if (have_prev)
                store_prev(p, p + 1);
            floatx4 acc[2] = {floatx4{0.0f, 0.0f, 0.0f, 0.0f}, floatx4{0.0f, 0.0f, 0.0f, 0.0f}};
            // the FP8 operands of four k-steps of both steps; the next group's
            // are requested before this group's conversions and products
            auto operands = [&](int k0, v2i(&a)[2][4]) {
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const uint8_t *tb = ring + (2 * p + h) * kTileBytes;
#pragma unroll
                    for (int k = 0; k < 4; k++)
                        a[h][k] = *(const v2i *)(tb + qoff[k0 + k]);
                }
            };
            v2i a[2][4];
            operands(0, a);
#pragma unroll
            for (int k0 = 0; k0 < 16; k0 += 4) {
                v2i an[2][4];
                if (k0 < 12)
                    operands(k0 + 4, an);
#pragma unroll
                for (int k = 0; k < 4; k++)
#pragma unroll
                    for (int h = 0; h < 2; h++)
                        acc[h] = mfma16x16x32(fp8x8_to_bf16x8(a[h][k]), as_bf16x8(qr[k0 + k]), acc[h]);
                if (k0 < 12) {
#pragma unroll
                    for (int h = 0; h < 2; h++)
#pragma unroll
                        for (int k = 0; k < 4; k++)
                            a[h][k] = an[h][k];
                }
            }
#pragma unroll
            for (int h = 0; h < 2; h++) {
                // a step whose every slot holds a selected token needs no mask
                if (__builtin_amdgcn_readfirstlane(vfull[2 * p + h])) {
#pragma unroll
                    for (int v = 0; v < 4; v++)
                        z[2 * p + h][v] = acc[h][v] * qk_log2;
                } else {
                    const int tt = 2 * (2 * p + h) + par;
                    const uint32_t mw = *(const uint32_t *)(vmask + 16 * tt + 4 * g);
#pragma unroll
                    for (int v = 0; v < 4; v++)
                        z[2 * p + h][v] = ((mw >> (8 * v)) & 0xFFu) ? acc[h][v] * qk_log2 : kNegInf;
                }
            }
        }

        // ================= the next unit: length and ids =================
        if (cu + 1 < uend)
            issue_len(cu + 1);
        else
            nu = units;

        // ================= maxima and softmax over the chunk =================
        {
            PIPE_LANE
            float mx = kNegInf;
#pragma unroll
            for (int st = 0; st < kMaxSteps; st++)
#pragma unroll
                for (int v = 0; v < 4; v++)
                    mx = __builtin_fmaxf(mx, z[st][v]);
            mx = max_xor32(max_xor16(mx));
            if (g == 0)
                wmax[wave][n16] = mx;
        }
        lds_barrier(); // wave maxima (every wave is past its QK: the vmask reads are done)
        float m;
        u32x2 pk[kMaxSteps];
        {
        PIPE_LANE
        m = __builtin_fmaxf(wmax[2 * ht][n16], wmax[2 * ht + 1][n16]);
        const float m_use = (m == kNegInf) ? 0.0f : m;
#pragma unroll
        for (int st = 0; st < kMaxSteps; st++) {
            float p4[4];
#pragma unroll
            for (int v = 0; v < 4; v++)
                p4[v] = __builtin_amdgcn_exp2f(z[st][v] - m_use);
            float ts = (p4[0] + p4[1]) + (p4[2] + p4[3]);
            ts = add_xor32(add_xor16(ts));
            if (g == 0)
                tsum[2 * st + par][hl] = ts;
            pk[st].x = pack_bf16x2(p4[0], p4[1]);
            pk[st].y = pack_bf16x2(p4[2], p4[3]);
        }
        }

        // ================= P.V, pass 0 (steps 0-3) =================
        floatx4 o[kHt][kPvColTiles];
#pragma unroll
        for (int mt = 0; mt < kHt; mt++)
#pragma unroll
            for (int i = 0; i < kPvColTiles; i++)
                o[mt][i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        auto write_p = [&](int pass) {
            PIPE_LANE
#pragma unroll
            for (int sp = 0; sp < kStepsPerPass; sp++)
                *(u32x2 *)(pbuf + hl * kPRowBytes + 2 * (kStep * sp + 8 * g + 4 * par)) =
                    pk[pass * kStepsPerPass + sp];
        };
        auto pv_pass = [&](int pass) {
            PIPE_LANE
            const int kp = n16 >> 1;
            const int trrow = (kp < 4) ? 4 * g + kp : 16 + 4 * g + (kp - 4);
#pragma unroll
            for (int sp = 0; sp < kStepsPerPass; sp++) {
                const uint8_t *tb = ring + (pass * kStepsPerPass + sp) * kTileBytes;
                v2i raw[kPvColTiles];
#pragma unroll
                for (int i = 0; i < kPvColTiles; i++)
                    raw[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (lds_v2i *)(tb + tile_off(trrow, kPvColTiles * wave + i) + 8 * (n16 & 1)));
                bf16x8 pa[kHt];
#pragma unroll
                for (int mt = 0; mt < kHt; mt++)
                    pa[mt] = as_bf16x8(*(const u32x4 *)(pbuf + (mt * 16 + n16) * kPRowBytes +
                                                        2 * (kStep * sp + 8 * g)));
#pragma unroll
                for (int i = 0; i < kPvColTiles; i++) {
                    const bf16x8 va = fp8x8_to_bf16x8(raw[i]);
#pragma unroll
                    for (int mt = 0; mt < kHt; mt++)
                        o[mt][i] = mfma16x16x32(va, pa[mt], o[mt][i]);
                }
            }
        };
        // ================= the next unit: page lookups =================
        // (in flight through the first P.V pass; the copies need them after it)
        const bool more = finish_b();
        // the next unit's query, into the registers this unit's QK is done with
        // (unless the next unit is a chunk of the same row and head group)
        if (more && (nr != cr || nhg != chg))
            issue_q(qr);
        write_p(0);
        lds_barrier(); // P of pass 0 and every tile sum
        pv_pass(0);
        // page lookups and query retired before the copies go out (a wait for
        // the query after them would also wait for the copies)
        __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
        lds_barrier(); // pass 0's ring and P reads are done
        if (more && wave < kStepsPerPass)
            issue_tile();
        write_p(1);
        lds_barrier(); // P of pass 1
        pv_pass(1);
        lds_barrier(); // pass 1's ring reads are done
        if (more && wave >= kStepsPerPass)
            issue_tile();
        // l of each head: the token-tile sums in tile order (read here, at
        // their use: the next unit rewrites them only after its QK)
        float lh[kHt];
        {
        PIPE_LANE
#pragma unroll
        for (int mt = 0; mt < kHt; mt++) {
            float acc = 0.0f;
#pragma unroll
            for (int tt = 0; tt < kTokTiles; tt++)
                acc += tsum[tt][16 * mt + n16];
            lh[mt] = acc;
        }
        }

        // ================= this unit becomes the previous one =================
        have_prev = true;
        pr = cr;
        phg = chg;
        pc = cc;
        pnch = cnch;
        pm = m;
        plh = lh[ht];
#pragma unroll
        for (int mt = 0; mt < kHt; mt++) {
            const float sc = (cnch == 1) ? (lh[mt] > 0.0f ? kv_scale / lh[mt] : 0.0f) : 1.0f;
#pragma unroll
            for (int i = 0; i < kPvColTiles; i++) {
                pw[mt][i].x = pack_bf16x2(o[mt][i][0] * sc, o[mt][i][1] * sc);
                pw[mt][i].y = pack_bf16x2(o[mt][i][2] * sc, o[mt][i][3] * sc);
            }
        }
        if (!more)
            break;
        cu = nu;
        cr = nr;
        chg = nhg;
        cc = nc;
        cnch = nnch;
    }
    store_prev(0, kHt);
#undef PIPE_LANE
}

// Fold the per-chunk partials of every (row, head): one wave per head,
// kMergeHeads heads per workgroup, 8 latent columns per lane (the (m, l)
// pairs of a head are wave-uniform loads).
// The partial pointers carry no __restrict__, so the first batch's loads are
// not sunk below the row-length test: loads through const restrict pointers
// count as invariant and move freely.
constexpr int kMergeHeads = 4;
__global__ __launch_bounds__(kWave * kMergeHeads) void k_mla_merge(const uint16_t *part_o,
                                                                  const float2 *part_ml,
                                                                  const int32_t *__restrict__ seq_lens,
                                                                  uint16_t *__restrict__ out, int H,
                                                                  int top_k, int max_len, int nch_max,
                                                                  int hg_count, int G, float kv_scale)
{
    const int r = blockIdx.y;
    const int h = blockIdx.x * kMergeHeads + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (h >= H)
        return;
    const int hg = h / G;
    const int hl = h % G;
    const int d = (threadIdx.x % kWave) * kFoldCols;
    const int64_t pbase = ((int64_t)r * hg_count + hg) * nch_max * G + hl;
    FoldBatch b;
    // the first batch goes out before the row's chunk count is known (every
    // chunk up to nch_max has its place in the workspace)
    fold_load(part_o, part_ml, pbase, G, 0, nch_max - 1, d, b);
    __asm__ volatile("" ::: "memory"); // those loads stay ahead of the length load and test
    const int L = min(max(seq_lens[r], 0), max_len);
    const int n = min(top_k, L);
    const int nch = (n + kAttChunk - 1) / kAttChunk;
    if (nch <= 1)
        return;
    FoldState f;
    f.m = kNegInf;
    f.l = 0.0f;
#pragma unroll
    for (int i = 0; i < kFoldCols; i++)
        f.acc[i] = 0.0f;
    for (int c0 = 0; c0 < nch; c0 += kFoldBatch) {
        if (c0 > 0)
            fold_load(part_o, part_ml, pbase, G, c0, nch - 1, d, b);
        fold_step(c0, nch, b, f);
    }
    *(u32x4 *)(out + ((int64_t)r * H + h) * kLat + d) = fold_output(f, kv_scale);
}

// Compute units of the current device (cached per device).
static int device_cus()
{
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

int launch_mla_decode(const LaunchShape &ls, const uint16_t *q, const uint8_t *kv_cache,
                      const int32_t *block_tables, const int32_t *seq_lens, const int32_t *sel,
                      float kv_scale, float sm_scale, uint16_t *out, char *ws,
                      const Workspace &wl, hipStream_t stream, KTimer t_att, KTimer t_merge)
{
    const int nch_max = att_chunks(ls) > 0 ? att_chunks(ls) : 1;
    const float qk_log2 = (float)((double)sm_scale * (double)kv_scale * 1.4426950408889634074);
    uint16_t *part_o = (uint16_t *)(ws + wl.part_o);
    float2 *part_ml = (float2 *)(ws + wl.part_ml);
    // Heads per workgroup: the smallest of 16, 32 and 64 that still leaves at
    // most one workgroup per CU (a small batch spreads over more CUs, each
    // pulling a part of the query; a large batch gathers the latent rows
    // once per 64 heads). Results do not depend on the choice. The partials
    // of any of them fit the workspace, which is sized for groups of 64.
    const int64_t units = (int64_t)ls.num_rows * nch_max;
    int G = kAttHeads;
    if (units * ((ls.num_heads + 15) / 16) <= device_cus())
        G = 16;
    else if (units * ((ls.num_heads + 31) / 32) <= device_cus())
        G = 32;
    const int hgc = (ls.num_heads + G - 1) / G;
    const int cus = device_cus();
    if (G == kAttHeads && units * hgc > cus) {
        // more units than CUs: one workgroup per CU walks its units in turn
        // (the same results; the next unit's copies overlap this one's work)
        hipExtLaunchKernelGGL(k_mla_decode_pipe, dim3(cus), dim3(kAttThreads), 0, stream, t_att.start,
                              t_att.stop, 0u, q, kv_cache, block_tables, seq_lens, sel, part_o, part_ml,
                              out, ls.rows_per_seq, ls.num_heads, ls.top_k, ls.page_size, ls.max_blocks,
                              ls.num_pages, ls.max_len, kv_scale, qk_log2, nch_max, hgc,
                              (int)(units * hgc));
    } else {
        const dim3 grid(nch_max * hgc, ls.num_rows);
        auto kern = G == 16 ? k_mla_decode<16> : G == 32 ? k_mla_decode<32> : k_mla_decode<kAttHeads>;
        hipExtLaunchKernelGGL(kern, grid, dim3(kAttThreads), 0, stream, t_att.start, t_att.stop, 0u, q,
                              kv_cache, block_tables, seq_lens, sel, part_o, part_ml, out,
                              ls.rows_per_seq, ls.num_heads, ls.top_k, ls.page_size, ls.max_blocks,
                              ls.num_pages, ls.max_len, kv_scale, qk_log2, nch_max, hgc);
    }
    if (hipGetLastError() != hipSuccess)
        return -1;
    if (nch_max > 1) {
        hipExtLaunchKernelGGL(k_mla_merge, dim3((ls.num_heads + kMergeHeads - 1) / kMergeHeads, ls.num_rows),
                              dim3(kWave * kMergeHeads), 0, stream,
                              t_merge.start, t_merge.stop, 0u, part_o, part_ml, seq_lens, out,
                              ls.num_heads, ls.top_k, ls.max_len, nch_max, hgc, G, kv_scale);
        if (hipGetLastError() != hipSuccess)
            return -1;
    } else {
        for (hipEvent_t e : {t_merge.start, t_merge.stop})
            if (e != nullptr && hipEventRecord(e, stream) != hipSuccess)
                return -1;
    }
    return 0;
}

} // namespace dsa
