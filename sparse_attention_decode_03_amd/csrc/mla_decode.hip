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
//  - A row's selection is cut into chunks of 256 slots. One workgroup
//    (4 waves x 16 heads = 64 heads) handles one chunk: it walks the chunk in
//    steps of 32 tokens, gathering each token's 512-byte FP8 row through the
//    block table with coalesced 16-byte loads, dequantising it exactly to
//    bf16 (E4M3 is a subset of bf16; kv_scale is folded into the logit scale
//    and the output) and parking the 32 x 512 tile in LDS, token-major, in
//    padded rows that keep both operand reads below free of bank conflicts.
//  - QK: S^T[token, head] on 16x16x32 bf16 MFMA, the tile as A (k = latent
//    dim), Q as B (staged in LDS once per workgroup). The MFMA output leaves
//    each lane with eight tokens of one head, which are exactly the k-slots
//    of that lane's PV operand, so the probabilities never leave registers.
//  - Online softmax in fp32 (log2 domain, exp2), fixed-order reductions.
//  - PV: O[head, d] on 16x16x32 bf16 MFMA, P (bf16) as A, the tile as B read
//    through LDS transpose loads (ds_read_tr16_b64), fp32 accumulators.
//  - A row with one chunk writes its bf16 output directly. Otherwise every
//    chunk writes (m, l, O) partials and k_mla_merge folds them in chunk
//    order 0, 1, 2, ... with the same fp32 formula for every row.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kAttThreads = 256;
constexpr int kStep = 32;          // tokens per LDS tile
constexpr int kLat = 512;          // latent width
constexpr int kRowChunks = kLat / 8; // 16-byte chunks per bf16 latent row (64)
// LDS rows (a token's bf16 latent, or a head's bf16 query) are padded from
// 1024 to 1072 bytes (67 chunks). With a 48-byte pad, 16 consecutive rows read
// at one chunk start 12 words apart modulo the 64 banks (all distinct 4-word
// groups), and the 4 consecutive rows x 4 eight-byte segments of one
// transpose read land on 32 distinct banks. Addresses stay a lane base plus
// compile-time offsets.
constexpr int kRowStride = kRowChunks + 3; // in 16-byte chunks
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

__global__ __launch_bounds__(kAttThreads, 1) void k_mla_decode(
    const uint16_t *__restrict__ q, const uint8_t *__restrict__ kv,
    const int32_t *__restrict__ bt, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ sel, float *__restrict__ part_o, float2 *__restrict__ part_ml,
    uint16_t *__restrict__ out, int K, int H, int top_k, int ps, int max_blocks, int num_pages,
    int max_len, float kv_scale, float qk_log2, int nch_max, int hg_count)
{
    __shared__ u32x4 tile[kStep * kRowStride];      // bf16 tokens x latent, padded rows
    __shared__ u32x4 qlds[kAttHeads * kRowStride];  // bf16 Q of the 64 heads, padded rows
    __shared__ int rowidx[kAttChunk];               // latent row of each slot, -1 = skip

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
    const int h_base = hg * kAttHeads + wave * 16;

    if (n == 0) {
        if (c == 0) {
            for (int i = tid; i < kAttHeads * kLat; i += kAttThreads) {
                const int h = hg * kAttHeads + i / kLat;
                if (h < H)
                    out[((int64_t)r * H + h) * kLat + (i % kLat)] = 0;
            }
        }
        return;
    }
    if (c >= nch)
        return;
    const bool wave_active = h_base < H;
    const int slot0 = c * kAttChunk;
    const int slot_end = min(n, slot0 + kAttChunk);

    // ---- resolve the chunk's selected tokens to latent rows once ----
    {
        const int slot = slot0 + tid;
        int row = -1;
        if (slot < slot_end) {
            const int t = sel[(int64_t)r * top_k + slot];
            if (t >= 0 && t < L) {
                const int page = bt[(int64_t)s * max_blocks + t / ps];
                if (page >= 0 && page < num_pages)
                    row = page * ps + t % ps;
            }
        }
        rowidx[tid] = row;
    }

    // Q of the workgroup's 64 heads into LDS (padded head rows).
#pragma unroll
    for (int i = 0; i < kAttHeads * kRowChunks / kAttThreads; i++) {
        const int id = i * kAttThreads + tid;
        const int hh = id / kRowChunks;
        const int ch = id % kRowChunks;
        const int h = hg * kAttHeads + hh;
        // branch-free: load a valid row, zero it if the head is padding
        u32x4 v = *(const u32x4 *)(q + ((int64_t)r * H + min(h, H - 1)) * kLat + ch * 8);
        if (h >= H)
            v = u32x4{0u, 0u, 0u, 0u};
        qlds[hh * kRowStride + ch] = v;
    }
    __syncthreads();

    float m_run = kNegInf; // running max of the log2-domain logits (head n16)
    float l_run = 0.0f;    // running sum of exp2(z - m_run)
    floatx4 o[32];
#pragma unroll
    for (int nt = 0; nt < 32; nt++)
        o[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    const int tq = tid >> 5; // staging: tokens 4*tq .. 4*tq+3
    const int dc = tid & 31; //          latent bytes 16*dc .. 16*dc+15

    // One step's 32 FP8 rows into registers; two steps stay in flight.
    auto gather = [&](u32x4 (&raw)[4], int base) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int k = base - slot0 + 4 * tq + i;
            const int row = (k < kAttChunk) ? rowidx[k] : -1;
            // branch-free so the four loads issue back to back: a skipped
            // slot reads latent row 0 and is zeroed
            raw[i] = *(const u32x4 *)(kv + (int64_t)max(row, 0) * kLat + 16 * dc);
            if (row < 0)
                raw[i] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    // Dequantise (exact) into the bf16 LDS tile.
    auto stage = [&](const u32x4 (&raw)[4]) {
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
            tile[t * kRowStride + 2 * dc] = lo;
            tile[t * kRowStride + 2 * dc + 1] = hi;
        }
    };
    // QK, online softmax and PV over the staged tile of step `base`.
    auto compute = [&](int base) {
        // ---- QK: lane ends with head n16, tokens 8g + 4a + v ----
        // ---- QK: S^T[token][head], tile rows as A (token 16a + n16, k =
        // latent dims 32*ks + 8*g .. +7), Q as B (head wave*16 + n16); the
        // lane ends with head n16 and tokens 16a + 4g + v (v = 0..3) ----
        floatx4 sacc[2] = {floatx4{0.0f, 0.0f, 0.0f, 0.0f}, floatx4{0.0f, 0.0f, 0.0f, 0.0f}};
        {
            const u32x4 *qrow = qlds + (wave * 16 + n16) * kRowStride + g;
            const u32x4 *t0row = tile + n16 * kRowStride + g;
            const u32x4 *t1row = tile + (16 + n16) * kRowStride + g;
#pragma unroll
            for (int ks = 0; ks < 16; ks++) {
                const bf16x8 qv = as_bf16x8(qrow[4 * ks]);
                sacc[0] = mfma16x16x32(as_bf16x8(t0row[4 * ks]), qv, sacc[0]);
                sacc[1] = mfma16x16x32(as_bf16x8(t1row[4 * ks]), qv, sacc[1]);
            }
        }
        // ---- online softmax (log2 domain) ----
        float z[8];
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float v = sacc[j >> 2][j & 3] * qk_log2;
            z[j] = rowidx[base - slot0 + 16 * (j >> 2) + 4 * g + (j & 3)] >= 0 ? v : kNegInf;
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
        rs += __shfl_xor(rs, 16, kWave);
        rs += __shfl_xor(rs, 32, kWave);
        l_run = __builtin_fmaf(l_run, alpha, rs);
        // O rows are heads 4g + v: rescale them by their own alpha, only on a
        // step where some head's reference moved (otherwise every alpha is
        // exactly 1, or O is still zero, and the multiply changes nothing)
        const bool grew = __ballot(move && m_run != kNegInf) != 0;
        m_run = m_new;
        if (grew) {
            float av[4];
#pragma unroll
            for (int v = 0; v < 4; v++)
                av[v] = __shfl(alpha, 4 * g + v, kWave);
#pragma unroll
            for (int nt = 0; nt < 32; nt++) {
                o[nt][0] *= av[0];
                o[nt][1] *= av[1];
                o[nt][2] *= av[2];
                o[nt][3] *= av[3];
            }
        }
        u32x4 pw;
        pw.x = pack_bf16x2(p[0], p[1]);
        pw.y = pack_bf16x2(p[2], p[3]);
        pw.z = pack_bf16x2(p[4], p[5]);
        pw.w = pack_bf16x2(p[6], p[7]);
        const bf16x8 pa = as_bf16x8(pw);
        // ---- PV: O[head][d] += P[head][token] C[token][d]; P as A (k-slot
        // j <-> token 16(j>>2) + 4g + (j&3), exactly the tokens this lane's
        // softmax holds), the tile as B through two transpose loads of 4
        // consecutive rows each: lane n16 receives latent column 16*nt + n16 ----
        const char *tb = (const char *)tile;
        const char *p0 = tb + (4 * g + (n16 >> 2)) * (kRowStride * 16) + 8 * (n16 & 3);
        const char *p1 = p0 + 16 * (kRowStride * 16);
#pragma unroll
        for (int nt = 0; nt < 32; nt++) {
            const shortx4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p0 + 32 * nt));
            const shortx4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p1 + 32 * nt));
            typedef short shortx8 __attribute__((ext_vector_type(8)));
            const shortx8 bb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
            o[nt] = mfma16x16x32(pa, __builtin_bit_cast(bf16x8, bb), o[nt]);
        }
    };

    u32x4 ra[4], rb[4];
    gather(ra, slot0);
    if (slot0 + kStep < slot_end)
        gather(rb, slot0 + kStep);
    for (int base = slot0; base < slot_end; base += 2 * kStep) {
        stage(ra);
        __syncthreads();
        if (base + 2 * kStep < slot_end)
            gather(ra, base + 2 * kStep);
        if (wave_active)
            compute(base);
        __syncthreads();
        if (base + kStep >= slot_end)
            break;
        stage(rb);
        __syncthreads();
        if (base + 3 * kStep < slot_end)
            gather(rb, base + 3 * kStep);
        if (wave_active)
            compute(base + kStep);
        __syncthreads();
    }

    if (!wave_active)
        return;
    if (nch == 1) {
        float inv[4];
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const float lh = __shfl(l_run, 4 * g + v, kWave);
            inv[v] = lh > 0.0f ? kv_scale / lh : 0.0f;
        }
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int h = h_base + 4 * g + v;
            if (h < H) {
                uint16_t *orow = out + ((int64_t)r * H + h) * kLat;
#pragma unroll
                for (int nt = 0; nt < 32; nt++)
                    orow[16 * nt + n16] = f32_to_bf16_rne(o[nt][v] * inv[v]);
            }
        }
    } else {
        const int64_t pbase = (((int64_t)r * hg_count + hg) * nch_max + c) * kAttHeads;
        if (g == 0)
            part_ml[pbase + wave * 16 + n16] = float2{m_run, l_run};
#pragma unroll
        for (int v = 0; v < 4; v++) {
            float *prow = part_o + (pbase + wave * 16 + 4 * g + v) * kLat;
#pragma unroll
            for (int nt = 0; nt < 32; nt++)
                prow[16 * nt + n16] = o[nt][v];
        }
    }
}

// Fold the per-chunk partials of every (row, head) in chunk order.
__global__ __launch_bounds__(128) void k_mla_merge(const float *__restrict__ part_o,
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
    // then folded strictly in chunk order
    constexpr int kB = 8;
    for (int c0 = 0; c0 < nch; c0 += kB) {
        float2 ml[kB];
        floatx4 ov[kB];
#pragma unroll
        for (int k = 0; k < kB; k++) {
            // branch-free: chunks past the row's last re-read its last one
            const int64_t pi =
                (((int64_t)r * hg_count + hg) * nch_max + min(c0 + k, nch - 1)) * kAttHeads + hl;
            ml[k] = part_ml[pi];
            ov[k] = *(const floatx4 *)(part_o + pi * kLat + d);
        }
#pragma unroll
        for (int k = 0; k < kB; k++) {
            if (c0 + k >= nch)
                break;
            const float m_new = __builtin_fmaxf(m_acc, ml[k].x);
            if (m_new == kNegInf)
                continue;
            const float a = exp2f(m_acc - m_new);
            const float b = exp2f(ml[k].x - m_new);
            l_acc = __builtin_fmaf(ml[k].y, b, l_acc * a);
#pragma unroll
            for (int i = 0; i < 4; i++)
                acc[i] = __builtin_fmaf(ov[k][i], b, acc[i] * a);
            m_acc = m_new;
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
    float *part_o = (float *)(ws + wl.part_o);
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
