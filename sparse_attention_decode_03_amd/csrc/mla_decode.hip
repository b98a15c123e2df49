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
//  - A row's selection is cut into chunks of kAttChunk slots. One workgroup
//    of 4 waves covers one chunk for 64 heads. It walks the chunk in steps of
//    32 tokens: each token's 512-byte FP8 row is gathered through the block
//    table with coalesced 16-byte loads (two steps ahead), dequantised
//    exactly to bf16 (E4M3 is a subset of bf16; kv_scale is folded into the
//    logit scale and the output) and parked in one of two LDS tiles,
//    token-major, in padded rows that keep the operand reads below free of
//    bank conflicts. Two barriers per step.
//  - QK + softmax, split by heads: scoring wave w computes S^T[token, head]
//    for heads 16w..16w+15 on 16x16x32 bf16 MFMA, the tile as A and the query
//    (staged in LDS once per workgroup) as B. Online
//    softmax in fp32 (log2 domain, exp2, fixed-order reductions, lazy
//    rescale). The bf16 probabilities go to a small LDS buffer laid out in
//    the PV operand's k order (one 16-byte write, one 16-byte read).
//  - PV, split by latent columns: each of the 8 waves accumulates O[all 64
//    heads, its 64 columns] on 16x16x32 bf16 MFMA, P as A, the tile as B
//    through LDS transpose loads (ds_read_tr16_b64). Each wave thus reads an
//    eighth of the tile instead of all of it.
//  - Roles: waves 0-3 score (QK + softmax) while waves 4-7 dequantise and
//    stage the next tile and keep the gathers in flight; all 8 run PV. Two
//    waves per SIMD, so one role's waits hide behind the other's work.
//  - A row with one chunk writes its bf16 output directly. Otherwise every
//    chunk writes (m, l) in fp32 and its unnormalised O rounded to bf16 (the
//    precision of the output; half the partial traffic), and k_mla_merge
//    folds them in chunk order 0, 1, 2, ... with the same fp32 formula for
//    every row.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kAttThreads = 512; // 8 waves, two per SIMD
constexpr int kStep = 32;            // tokens per LDS tile
constexpr int kLat = 512;            // latent width
constexpr int kRowChunks = kLat / 8; // 16-byte chunks per bf16 latent row (64)
constexpr int kPvCols = kLat / (kAttThreads / kWave); // latent columns of one wave's PV (64)
constexpr int kPvTiles = kPvCols / 16;                // its 16-column MFMA tiles (4)
// LDS tile rows (a token's bf16 latent) are padded from 1024 to 1056 bytes
// (66 chunks): measured on gfx950 the fastest stride for the QK operand
// reads (16 rows at one 16-byte column per lane group), and within 10 % of
// the best for the PV transpose reads. Addresses stay a lane base plus
// compile-time offsets.
constexpr int kRowStride = kRowChunks + 2; // in 16-byte chunks
// Probability rows (one head, 32 bf16) are padded from 64 to 80 bytes: 16
// consecutive heads read at one 16-byte column hit 16 distinct 4-bank groups.
constexpr int kPRowBytes = 80;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

__global__ __launch_bounds__(kAttThreads, 1) void k_mla_decode(
    const uint16_t *__restrict__ q, const uint8_t *__restrict__ kv,
    const int32_t *__restrict__ bt, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ sel, uint16_t *__restrict__ part_o, float2 *__restrict__ part_ml,
    uint16_t *__restrict__ out, int K, int H, int top_k, int ps, int max_blocks, int num_pages,
    int max_len, float kv_scale, float qk_log2, int nch_max, int hg_count)
{
    __shared__ u32x4 tile[2][kStep * kRowStride];        // bf16 tokens x latent, padded rows
    __shared__ u32x4 qlds[kAttHeads * kRowStride];       // bf16 query of the 64 heads, padded
    __shared__ __align__(16) uint8_t pbuf[kAttHeads * kPRowBytes]; // bf16 P, PV k order
    __shared__ float alds[kAttHeads];                    // per-head rescale factors
    __shared__ float2 mlds[kAttHeads];                   // per-head (m, l) at the end
    __shared__ int rowidx[kAttChunk];                    // latent row of each slot, -1 = skip
    __shared__ int resc_step;                            // last step whose O needs a rescale

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int g = lane >> 4;
    const int n16 = lane & 15;
    const int r = blockIdx.y;
    const int c = blockIdx.x % nch_max;
    const int hg = blockIdx.x / nch_max;
    const int s = r / K;
    const int L = min(max(seq_lens[r], 0), max_len);
    const int n = min(top_k, L);
    const int nch = (n + kAttChunk - 1) / kAttChunk;
    const int h0 = hg * kAttHeads;              // first head of the group
    const int nh = min(kAttHeads, H - h0);      // heads of the group that exist
    const int hq = h0 + (wave & 3) * 16 + n16;  // this lane's head in QK (waves 0-3)
    const bool qk_active = wave < 4 && wave * 16 < nh; // a scoring wave whose heads exist
    const bool producer = wave >= 4;            // waves 4-7 gather and stage the tiles

    if (n == 0) {
        if (c == 0) {
            for (int i = tid; i < kAttHeads * kLat; i += kAttThreads) {
                const int h = h0 + i / kLat;
                if (h < H)
                    out[((int64_t)r * H + h) * kLat + (i % kLat)] = 0;
            }
        }
        return;
    }
    if (c >= nch)
        return;
    const int slot0 = c * kAttChunk;
    const int nslots = min(n - slot0, kAttChunk);
    const int nsteps = (nslots + kStep - 1) / kStep;

    // ---- resolve the chunk's selected tokens to latent rows once ----
    for (int k = tid; k < kAttChunk; k += kAttThreads) {
        int row = -1;
        if (k < nslots) {
            const int t = sel[(int64_t)r * top_k + slot0 + k];
            if (t >= 0 && t < L) {
                const int page = bt[(int64_t)s * max_blocks + t / ps];
                if (page >= 0 && page < num_pages)
                    row = page * ps + t % ps;
            }
        }
        rowidx[k] = row;
    }
    if (tid == 0)
        resc_step = -1;

    // ---- query of the group's 64 heads into LDS (padded head rows);
    // branch-free, a missing head loads head H-1 and is zeroed ----
#pragma unroll
    for (int i = 0; i < kAttHeads * kRowChunks / kAttThreads; i++) {
        const int id = i * kAttThreads + tid;
        const int hh = id / kRowChunks;
        const int ch = id % kRowChunks;
        const int h = h0 + hh;
        u32x4 v = *(const u32x4 *)(q + ((int64_t)r * H + min(h, H - 1)) * kLat + ch * 8);
        if (h >= H)
            v = u32x4{0u, 0u, 0u, 0u};
        qlds[hh * kRowStride + ch] = v;
    }

    float m_run = kNegInf; // reference max of the log2-domain logits (head hq)
    float l_run = 0.0f;    // this lane's share of sum exp2(z - m_run)
    floatx4 o[4][kPvTiles]; // O[head 16*mt + 4g + v][column kPvCols*wave + 16*nt + n16]
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int nt = 0; nt < kPvTiles; nt++)
            o[mt][nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    int mt_count = (nh + 15) / 16; // head tiles that exist

    const int ptid = tid - 4 * kWave; // staging thread among waves 4-7
    const int tq = (ptid >> 5) & 7;   // staging: tokens 4*tq .. 4*tq+3
    const int dc = ptid & 31;         //          latent bytes 16*dc .. 16*dc+15

    // One step's 32 FP8 rows into registers; two steps stay in flight.
    auto gather = [&](u32x4 (&raw)[4], int step) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int k = step * kStep + 4 * tq + i;
            const int row = (k < kAttChunk) ? rowidx[k] : -1;
            // branch-free so the four loads issue back to back: a skipped
            // slot reads latent row 0 and is zeroed
            raw[i] = *(const u32x4 *)(kv + (int64_t)max(row, 0) * kLat + 16 * dc);
            if (row < 0)
                raw[i] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    // Dequantise (exact) into LDS tile b.
    auto stage = [&](const u32x4 (&raw)[4], int b) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int t = 4 * tq + i;
            u32x4 lo, hi;
            lo.x = e4m3x2_to_bf16x2_exact<false>(raw[i].x);
            lo.y = e4m3x2_to_bf16x2_exact<true>(raw[i].x);
            lo.z = e4m3x2_to_bf16x2_exact<false>(raw[i].y);
            lo.w = e4m3x2_to_bf16x2_exact<true>(raw[i].y);
            hi.x = e4m3x2_to_bf16x2_exact<false>(raw[i].z);
            hi.y = e4m3x2_to_bf16x2_exact<true>(raw[i].z);
            hi.z = e4m3x2_to_bf16x2_exact<false>(raw[i].w);
            hi.w = e4m3x2_to_bf16x2_exact<true>(raw[i].w);
            // lanes dc and dc + 8 would hit the same banks with the chunk
            // pair in order; the upper eight of every sixteen write it swapped
            const int sw = (dc >> 3) & 1;
            tile[b][t * kRowStride + 2 * dc + sw] = sw ? hi : lo;
            tile[b][t * kRowStride + 2 * dc + 1 - sw] = sw ? lo : hi;
        }
    };

    // QK and online softmax of step `step` (tile b) for this wave's heads;
    // leaves P in pbuf and, on a step where a reference moved, the alphas.
    auto qk_softmax = [&](int step, int b) {
        floatx4 sacc[2] = {floatx4{0.0f, 0.0f, 0.0f, 0.0f}, floatx4{0.0f, 0.0f, 0.0f, 0.0f}};
        // A: tile rows n16 and 16 + n16, k = latent dims 32*ks + 8*g .. +7;
        // B: query of head wave*16 + n16 with the same k order. Operands of
        // four k-steps are read ahead of their products.
        const u32x4 *t0row = tile[b] + n16 * kRowStride + g;
        const u32x4 *t1row = tile[b] + (16 + n16) * kRowStride + g;
        const u32x4 *qrow = qlds + (wave * 16 + n16) * kRowStride + g;
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
            u32x4 a0[4], a1[4], qb[4];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                a0[j] = t0row[4 * (k0 + j)];
                a1[j] = t1row[4 * (k0 + j)];
                qb[j] = qrow[4 * (k0 + j)];
            }
#pragma unroll
            for (int j = 0; j < 4; j++) {
                sacc[0] = mfma16x16x32(as_bf16x8(a0[j]), as_bf16x8(qb[j]), sacc[0]);
                sacc[1] = mfma16x16x32(as_bf16x8(a1[j]), as_bf16x8(qb[j]), sacc[1]);
            }
        }
        // lane: head hq, tokens 16*(j>>2) + 4g + (j&3) for j = 0..7
        float z[8];
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float v = sacc[j >> 2][j & 3] * qk_log2;
            z[j] = rowidx[step * kStep + 16 * (j >> 2) + 4 * g + (j & 3)] >= 0 ? v : kNegInf;
            mx = __builtin_fmaxf(mx, z[j]);
        }
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, kWave));
        // The reference max moves only when the step's max exceeds it by
        // more than kRescaleSlack (log2 units): then p <= 2^kRescaleSlack, so
        // fp32 sums and bf16 probabilities stay well scaled, and O is
        // rescaled only on rare steps. The rule is a function of the row's
        // data alone, so results stay bit-reproducible; the partial state
        // (m_ref, l, O) merges exactly as with the true max.
        const bool move = mx > m_run + kRescaleSlack;
        const float m_new = move ? mx : m_run;
        const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float p[8];
        float rs = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            p[j] = exp2f(z[j] - m_use);
            rs += p[j];
        }
        l_run = __builtin_fmaf(l_run, alpha, rs);
        // every step leaves its alphas (1 where nothing moved); the PV waves
        // apply them only on a step marked here
        if (g == 0)
            alds[wave * 16 + n16] = alpha;
        if (__ballot(move && m_run != kNegInf) != 0 && lane == 0)
            resc_step = step;
        m_run = m_new;
        u32x4 pw;
        pw.x = pack_bf16x2(p[0], p[1]);
        pw.y = pack_bf16x2(p[2], p[3]);
        pw.z = pack_bf16x2(p[4], p[5]);
        pw.w = pack_bf16x2(p[6], p[7]);
        *(u32x4 *)(pbuf + (wave * 16 + n16) * kPRowBytes + 16 * g) = pw;
    };

    // PV of step `step` (tile b): O[heads, this wave's kPvCols columns]. P as
    // A (k-slot j <-> token 16(j>>2) + 4g + (j&3)), the tile as B through two
    // transpose loads of 4 consecutive rows each: lane n16 receives column
    // kPvCols*wave + 16*nt + n16, rows 4g..4g+3 and 16+4g..16+4g+3.
    auto pv = [&](int step, int b) {
        const bool resc = resc_step == step;
        const char *tb = (const char *)tile[b];
        const char *p0 = tb + (4 * g + (n16 >> 2)) * (kRowStride * 16) + 8 * (n16 & 3) +
                         2 * kPvCols * wave;
        const char *p1 = p0 + 16 * (kRowStride * 16);
        shortx8 vb[kPvTiles];
#pragma unroll
        for (int nt = 0; nt < kPvTiles; nt++) {
            const shortx4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p0 + 32 * nt));
            const shortx4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p1 + 32 * nt));
            vb[nt] = shortx8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        }
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
            if (mt < mt_count) {
                const bf16x8 pa = as_bf16x8(*(const u32x4 *)(pbuf + (16 * mt + n16) * kPRowBytes + 16 * g));
                if (resc) {
                    const floatx4 av = *(const floatx4 *)(alds + 16 * mt + 4 * g);
#pragma unroll
                    for (int nt = 0; nt < kPvTiles; nt++) {
                        o[mt][nt][0] *= av[0];
                        o[mt][nt][1] *= av[1];
                        o[mt][nt][2] *= av[2];
                        o[mt][nt][3] *= av[3];
                    }
                }
#pragma unroll
                for (int nt = 0; nt < kPvTiles; nt++)
                    o[mt][nt] = mfma16x16x32(pa, __builtin_bit_cast(bf16x8, vb[nt]), o[mt][nt]);
            }
        }
    };

    __syncthreads(); // rowidx and resc_step visible
    u32x4 ra[4], rb[4];
    if (producer) {
        gather(ra, 0);
        if (nsteps > 1)
            gather(rb, 1);
        stage(ra, 0);
        if (nsteps > 2)
            gather(ra, 2);
    }
    // step i computes from tile i & 1; while waves 0-3 score step i, waves
    // 4-7 stage step i + 1 into the other tile and gather the rows of step
    // i + 3; then all eight waves run PV of step i
    for (int i = 0; i < nsteps; i += 2) {
        __syncthreads(); // tile 0 holds step i; PV of step i - 1 is done
        if (qk_active)
            qk_softmax(i, 0);
        if (producer && i + 1 < nsteps) {
            stage(rb, 1);
            if (i + 3 < nsteps)
                gather(rb, i + 3);
        }
        __syncthreads(); // P of step i visible
        pv(i, 0);
        if (i + 1 >= nsteps)
            break;
        __syncthreads(); // tile 1 holds step i + 1; PV of step i is done
        if (qk_active)
            qk_softmax(i + 1, 1);
        if (producer && i + 2 < nsteps) {
            stage(ra, 0);
            if (i + 4 < nsteps)
                gather(ra, i + 4);
        }
        __syncthreads();
        pv(i + 1, 1);
    }

    // ---- per-head (m, l): the four lanes of a head hold shares of l ----
    const float l_tot = l_run + __shfl_xor(l_run, 16, kWave);
    const float l_all = l_tot + __shfl_xor(l_tot, 32, kWave);
    if (qk_active && g == 0)
        mlds[wave * 16 + n16] = float2{m_run, l_all};
    __syncthreads();

    if (nch == 1) {
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
            if (mt >= mt_count)
                break;
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int hl = 16 * mt + 4 * g + v;
                const int h = h0 + hl;
                if (h < H) {
                    const float lh = mlds[hl].y;
                    const float inv = lh > 0.0f ? kv_scale / lh : 0.0f;
                    uint16_t *orow = out + ((int64_t)r * H + h) * kLat + kPvCols * wave + n16;
#pragma unroll
                    for (int nt = 0; nt < kPvTiles; nt++)
                        orow[16 * nt] = f32_to_bf16_rne(o[mt][nt][v] * inv);
                }
            }
        }
    } else {
        const int64_t pbase = (((int64_t)r * hg_count + hg) * nch_max + c) * kAttHeads;
        if (qk_active && g == 0)
            part_ml[pbase + wave * 16 + n16] = float2{m_run, l_all};
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
            if (mt >= mt_count)
                break;
#pragma unroll
            for (int v = 0; v < 4; v++) {
                uint16_t *prow = part_o + (pbase + 16 * mt + 4 * g + v) * kLat + kPvCols * wave + n16;
#pragma unroll
                for (int nt = 0; nt < kPvTiles; nt++)
                    prow[16 * nt] = f32_to_bf16_rne(o[mt][nt][v]);
            }
        }
    }
}

// Fold the per-chunk partials of every (row, head) in chunk order.
__global__ __launch_bounds__(128) void k_mla_merge(const uint16_t *__restrict__ part_o,
                                                   const float2 *__restrict__ part_ml,
                                                   const int32_t *__restrict__ seq_lens,
                                                   uint16_t *__restrict__ out, int H, int top_k,
                                                   int max_len, int nch_max, int hg_count,
                                                   float kv_scale)
{
    const int r = blockIdx.y;
    const int h = blockIdx.x;
    const int L = min(max(seq_lens[r], 0), max_len);
    const int n = min(top_k, L);
    const int nch = (n + kAttChunk - 1) / kAttChunk;
    if (nch <= 1)
        return;
    const int hg = h / kAttHeads;
    const int hl = h % kAttHeads;
    const int d = threadIdx.x * 4;
    float m_acc = kNegInf, l_acc = 0.0f;
    floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    // partials are loaded in unrolled batches (independent loads in flight),
    // then folded strictly in chunk order; straight-line code with selects,
    // so the batch stays in registers
    constexpr int kB = 16;
    for (int c0 = 0; c0 < nch; c0 += kB) {
        float2 ml[kB];
        floatx4 ov[kB];
#pragma unroll
        for (int k = 0; k < kB; k++) {
            // branch-free: chunks past the row's last re-read its last one
            const int64_t pi =
                (((int64_t)r * hg_count + hg) * nch_max + min(c0 + k, nch - 1)) * kAttHeads + hl;
            ml[k] = part_ml[pi];
            const u32x2 pk = *(const u32x2 *)(part_o + pi * kLat + d);
            ov[k] = floatx4{__uint_as_float(pk.x << 16), __uint_as_float(pk.x & 0xFFFF0000u),
                            __uint_as_float(pk.y << 16), __uint_as_float(pk.y & 0xFFFF0000u)};
        }
#pragma unroll
        for (int k = 0; k < kB; k++) {
            const float m_new = __builtin_fmaxf(m_acc, ml[k].x);
            // a chunk past the last, or one with nothing selected so far,
            // leaves the state untouched
            const bool use = (c0 + k < nch) && (m_new != kNegInf);
            const float a = use ? exp2f(m_acc - m_new) : 1.0f;
            const float b = use ? exp2f(ml[k].x - m_new) : 0.0f;
            l_acc = use ? __builtin_fmaf(ml[k].y, b, l_acc * a) : l_acc;
#pragma unroll
            for (int i = 0; i < 4; i++)
                acc[i] = use ? __builtin_fmaf(ov[k][i], b, acc[i] * a) : acc[i];
            m_acc = use ? m_new : m_acc;
        }
    }
    const float inv = l_acc > 0.0f ? kv_scale / l_acc : 0.0f;
    uint16_t *orow = out + ((int64_t)r * H + h) * kLat + d;
    u32x2 packed;
    packed.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    packed.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *(u32x2 *)orow = packed;
}

int launch_mla_decode(const LaunchShape &ls, const uint16_t *q, const uint8_t *kv_cache,
                      const int32_t *block_tables, const int32_t *seq_lens, const int32_t *sel,
                      float kv_scale, float sm_scale, uint16_t *out, char *ws,
                      const Workspace &wl, hipStream_t stream)
{
    const int nch_max = att_chunks(ls) > 0 ? att_chunks(ls) : 1;
    const int hgc = att_head_groups(ls);
    const float qk_log2 = (float)((double)sm_scale * (double)kv_scale * 1.4426950408889634074);
    uint16_t *part_o = (uint16_t *)(ws + wl.part_o);
    float2 *part_ml = (float2 *)(ws + wl.part_ml);
    hipLaunchKernelGGL(k_mla_decode, dim3(nch_max * hgc, ls.num_rows), dim3(kAttThreads), 0,
                       stream, q, kv_cache, block_tables, seq_lens, sel, part_o, part_ml, out,
                       ls.rows_per_seq, ls.num_heads, ls.top_k, ls.page_size, ls.max_blocks,
                       ls.num_pages, ls.max_len, kv_scale, qk_log2, nch_max, hgc);
    if (hipGetLastError() != hipSuccess)
        return -1;
    if (nch_max > 1) {
        hipLaunchKernelGGL(k_mla_merge, dim3(ls.num_heads, ls.num_rows), dim3(128), 0, stream,
                           part_o, part_ml, seq_lens, out, ls.num_heads, ls.top_k, ls.max_len,
                           nch_max, hgc, kv_scale);
        if (hipGetLastError() != hipSuccess)
            return -1;
    }
    return 0;
}

} // namespace dsa
