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
//    of 8 waves covers one chunk for a group of G heads (16, 32 or 64), in
//    steps of 32 tokens. Each token's 512-byte FP8 row is gathered through
//    the block table with
//    coalesced 16-byte loads, dequantised exactly to bf16 (E4M3 is a subset
//    of bf16; kv_scale is folded into the logit scale and the output) and
//    parked token-major in one of three LDS tiles, in padded rows that keep
//    the operand reads below free of bank conflicts.
//  - Two roles, one barrier per step. Waves 0-3 score: wave w holds the
//    query of heads 16w..16w+15 in registers and computes S^T[token, head]
//    on 16x16x32 bf16 MFMA (the tile as A, the query as B), then the online
//    softmax in fp32 (log2 domain, exp2, fixed-order reductions, lazy
//    rescale); the bf16 probabilities go to a small LDS buffer in the PV
//    operand's k order. Waves 4-7 accumulate: wave v holds O[G heads,
//    latent columns 128v..128v+127] and runs PV on 16x16x32 bf16 MFMA (P as
//    A, the tile as B through LDS transpose loads, ds_read_tr16_b64); they
//    also dequantise and stage the tiles and keep the gathers in flight.
//    While the scoring waves work on step i + 1, the accumulating waves run
//    PV of step i and stage step i + 2, so the matrix cores of every SIMD
//    see both products at once. Each result element is still produced by
//    the same operations in the same order, step after step.
//  - A row with one chunk writes its bf16 output directly. Otherwise every
//    chunk writes (m, l) in fp32 and its unnormalised O rounded to bf16 (the
//    precision of the output; half the partial traffic), and k_mla_merge
//    folds them in chunk order 0, 1, 2, ... with the same fp32 formula for
//    every row.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kAttThreads = 512;  // 8 waves, two per SIMD: one scoring, one accumulating
constexpr int kStep = 32;            // tokens per LDS tile
constexpr int kTiles = 3;            // tiles in LDS: scored, accumulated, being staged
constexpr int kLat = 512;            // latent width
constexpr int kRowChunks = kLat / 8; // 16-byte chunks per bf16 latent row (64)
constexpr int kPvCols = kLat / 4;    // latent columns of one accumulating wave (128)
constexpr int kPvTiles = kPvCols / 16; // its 16-column MFMA tiles (8)
constexpr int kMaxSteps = kAttChunk / kStep;
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
constexpr int kGatherDepth = 4;   // gather lookahead in steps, 16- and 32-head groups
constexpr int kGatherDepth64 = 2; // and 64-head groups

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// G: heads per workgroup (16, 32 or 64; scoring waves past G / 16 idle).
// Each head's arithmetic is the same whichever heads share its workgroup (a
// head whose reference did not move rescales by exactly 1), so G changes
// where the work runs, never a result.
// kv carries no __restrict__: loads through a const restrict pointer count as
// invariant, and the compiler then sinks the prologue's gathers past the
// barriers to just before their use, where the stage waits a full memory
// round trip for them.
template <int G>
__global__ __launch_bounds__(kAttThreads, 1) void k_mla_decode(
    const uint16_t *__restrict__ q, const uint8_t *kv,
    const int32_t *__restrict__ bt, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ sel, uint16_t *__restrict__ part_o, float2 *__restrict__ part_ml,
    uint16_t *__restrict__ out, int K, int H, int top_k, int ps, int max_blocks, int num_pages,
    int max_len, float kv_scale, float qk_log2, int nch_max, int hg_count)
{
    __shared__ u32x4 tile[kTiles][kStep * kRowStride];   // bf16 tokens x latent, padded rows
    __shared__ __align__(16) uint8_t pbuf[2][G * kPRowBytes]; // bf16 P, PV k order
    __shared__ __align__(16) float alds[2][G];   // per-head rescale factors
    __shared__ float2 mlds[G];                   // per-head (m, l) at the end
    __shared__ int rowidx[kAttChunk];                    // latent row of each slot, -1 = skip
    __shared__ int resc[kMaxSteps];                      // step s: O needs its alphas

    constexpr int kHt = G / 16; // 16-head MFMA tiles of the group
    // steps of gathers in flight: as deep as the accumulators leave registers
    // for (each step is 16 VGPRs per accumulating lane; 64 heads keep 128 in O)
    constexpr int kDepth = G == 64 ? kGatherDepth64 : kGatherDepth;
    static_assert(kHt >= 1 && kHt <= 4, "one scoring wave per 16 heads");
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
    if (tid < kMaxSteps)
        resc[tid] = 0;
    // P rows of heads that no scoring wave covers stay zero
    for (int i = tid; i < 2 * G * kPRowBytes / 16; i += kAttThreads)
        ((u32x4 *)pbuf)[i] = u32x4{0u, 0u, 0u, 0u};

    if (wave < 4) {
        // ================= scoring waves: QK + online softmax =================
        const int hl = wave * 16 + n16; // this lane's head within the group
        const bool active = wave < kHt && wave * 16 < nh;
        // query of head hl, latent dims 32 ks + 8 g .. +7 (the B operand).
        // A lane past the group's last head scores with head H-1's query:
        // its results are never stored, and it cannot change another head's
        // (its reference moves exactly when head H-1's does, and an unmoved
        // head rescales by exactly 1). Nothing reads the loads before the
        // first product, so they stay in flight through the prologue.
        u32x4 qr[16];
        if (active) {
            const uint16_t *qrow = q + ((int64_t)r * H + min(h0 + hl, H - 1)) * kLat + 8 * g;
#pragma unroll
            for (int ks = 0; ks < 16; ks++)
                qr[ks] = *(const u32x4 *)(qrow + 32 * ks);
        }
        float m_run = kNegInf; // reference max of the log2-domain logits (head hl)
        float l_run = 0.0f;    // this lane's share of sum exp2(z - m_run)

        // QK and online softmax of one step; leaves P and the alphas in
        // buffer step & 1 and marks the step when a reference moved
        auto qk_softmax = [&](int step) {
            const u32x4 *tb = tile[step % kTiles];
            floatx4 sacc[2] = {floatx4{0.0f, 0.0f, 0.0f, 0.0f}, floatx4{0.0f, 0.0f, 0.0f, 0.0f}};
            // A: tile rows n16 and 16 + n16, k = latent dims 32 ks + 8 g .. +7.
            // Software-pipelined in groups of four k-steps: the operands of
            // group k0 + 1 are requested before the products of group k0, so
            // the LDS latency hides behind the matrix core.
            const u32x4 *t0row = tb + n16 * kRowStride + g;
            const u32x4 *t1row = tb + (16 + n16) * kRowStride + g;
            u32x4 a[2][8];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                a[0][2 * j] = t0row[4 * j];
                a[0][2 * j + 1] = t1row[4 * j];
            }
#pragma unroll
            for (int k0 = 0; k0 < 4; k0++) {
                if (k0 + 1 < 4) {
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        a[(k0 + 1) & 1][2 * j] = t0row[4 * (4 * (k0 + 1) + j)];
                        a[(k0 + 1) & 1][2 * j + 1] = t1row[4 * (4 * (k0 + 1) + j)];
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    sacc[0] = mfma16x16x32(as_bf16x8(a[k0 & 1][2 * j]), as_bf16x8(qr[4 * k0 + j]), sacc[0]);
                    sacc[1] = mfma16x16x32(as_bf16x8(a[k0 & 1][2 * j + 1]), as_bf16x8(qr[4 * k0 + j]), sacc[1]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // lane: head hl, tokens 16*(j>>2) + 4g + (j&3) for j = 0..7
            float z[8];
            float mx = kNegInf;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const float v = sacc[j >> 2][j & 3] * qk_log2;
                z[j] = rowidx[step * kStep + 16 * (j >> 2) + 4 * g + (j & 3)] >= 0 ? v : kNegInf;
                mx = __builtin_fmaxf(mx, z[j]);
            }
            mx = max_xor32(max_xor16(mx));
            // The reference max moves only when the step's max exceeds it by
            // more than kRescaleSlack (log2 units): then p <= 2^kRescaleSlack,
            // so fp32 sums and bf16 probabilities stay well scaled, and O is
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
            if (g == 0)
                alds[step & 1][hl] = alpha;
            if (__ballot(move && m_run != kNegInf) != 0 && lane == 0)
                resc[step] = 1;
            m_run = m_new;
            u32x4 pw;
            pw.x = pack_bf16x2(p[0], p[1]);
            pw.y = pack_bf16x2(p[2], p[3]);
            pw.z = pack_bf16x2(p[4], p[5]);
            pw.w = pack_bf16x2(p[6], p[7]);
            *(u32x4 *)(pbuf[step & 1] + hl * kPRowBytes + 16 * g) = pw;
        };

        __syncthreads(); // rowidx, resc cleared
        __syncthreads(); // tile 0 staged
        if (active)
            qk_softmax(0);
        __syncthreads(); // P of step 0, tile 1 staged
        for (int i = 0; i < nsteps; i++) {
            if (active && i + 1 < nsteps)
                qk_softmax(i + 1);
            __syncthreads();
        }
        // per-head (m, l): the four lanes of a head hold shares of l
        const float l_all = add_xor32(add_xor16(l_run));
        if (active && g == 0) {
            mlds[hl] = float2{m_run, l_all};
            if (nch > 1) {
                const int64_t pbase = (((int64_t)r * hg_count + hg) * nch_max + c) * G;
                part_ml[pbase + hl] = float2{m_run, l_all};
            }
        }
        __syncthreads(); // mlds
        return;
    }

    // ================= accumulating waves: gather, stage, PV =================
    const int v = wave - 4;
    const int ptid = tid - 4 * kWave; // 0..255
    const int tq = ptid >> 5;         // staging: tokens 4 tq .. 4 tq + 3
    const int dc = ptid & 31;         //          latent bytes 16 dc .. 16 dc + 15
    floatx4 o[kHt][kPvTiles]; // O[head 16 mt + n16][columns kPvCols v + 16 nt + 4 g + e]
#pragma unroll
    for (int mt = 0; mt < kHt; mt++)
#pragma unroll
        for (int nt = 0; nt < kPvTiles; nt++)
            o[mt][nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // One step's 32 FP8 rows into registers (slot indices first, then the
    // four loads back to back; a skipped slot reads latent row 0 and is
    // zeroed when staged, so nothing waits on the loads here).
    auto gather = [&](u32x4 (&raw)[4], int step) {
        int row[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int k = step * kStep + 4 * tq + i;
            row[i] = (k < kAttChunk) ? rowidx[k] : -1;
        }
#pragma unroll
        for (int i = 0; i < 4; i++)
            raw[i] = *(const u32x4 *)(kv + (int64_t)max(row[i], 0) * kLat + 16 * dc);
    };
    // Dequantise (exact) into the tile of `step`.
    auto stage = [&](const u32x4 (&raw)[4], int step) {
        u32x4 *tb = tile[step % kTiles];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int t = 4 * tq + i;
            const int k = step * kStep + t;
            const bool skip = k >= kAttChunk || rowidx[k] < 0;
            const u32x4 w = skip ? u32x4{0u, 0u, 0u, 0u} : raw[i];
            u32x4 lo, hi;
            lo.x = e4m3x2_to_bf16x2_exact<false>(w.x);
            lo.y = e4m3x2_to_bf16x2_exact<true>(w.x);
            lo.z = e4m3x2_to_bf16x2_exact<false>(w.y);
            lo.w = e4m3x2_to_bf16x2_exact<true>(w.y);
            hi.x = e4m3x2_to_bf16x2_exact<false>(w.z);
            hi.y = e4m3x2_to_bf16x2_exact<true>(w.z);
            hi.z = e4m3x2_to_bf16x2_exact<false>(w.w);
            hi.w = e4m3x2_to_bf16x2_exact<true>(w.w);
            // lanes dc and dc + 8 would hit the same banks with the chunk
            // pair in order; the upper eight of every sixteen write it swapped
            const int sw = (dc >> 3) & 1;
            tb[t * kRowStride + 2 * dc + sw] = sw ? hi : lo;
            tb[t * kRowStride + 2 * dc + 1 - sw] = sw ? lo : hi;
        }
    };
    // PV of one step, transposed: O^T[this wave's columns, heads] += V^T P^T.
    // The tile as A through two transpose loads of 4 consecutive rows each
    // (lane n16 receives column kPvCols v + 16 nt + n16, rows 4g..4g+3 and
    // 16+4g..16+4g+3, i.e. k-slot j <-> token 16(j>>2) + 4g + (j&3)), P as B
    // in the same k order. A lane ends with 4 consecutive columns of one
    // head: one rescale factor per head tile, 8-byte output stores.
    auto pv = [&](int step) {
        const bool rs = resc[step] != 0;
        const char *tb = (const char *)tile[step % kTiles];
        const uint8_t *pb = pbuf[step & 1];
        const char *p0 = tb + (4 * g + (n16 >> 2)) * (kRowStride * 16) + 8 * (n16 & 3) +
                         2 * kPvCols * v;
        const char *p1 = p0 + 16 * (kRowStride * 16);
        if (rs) {
#pragma unroll
            for (int mt = 0; mt < kHt; mt++) {
                const float a = alds[step & 1][16 * mt + n16];
#pragma unroll
                for (int nt = 0; nt < kPvTiles; nt++) {
                    o[mt][nt][0] *= a;
                    o[mt][nt][1] *= a;
                    o[mt][nt][2] *= a;
                    o[mt][nt][3] *= a;
                }
            }
        }
        // every operand of the step is requested before the first product
        bf16x8 pa[4];
#pragma unroll
        for (int mt = 0; mt < kHt; mt++)
            pa[mt] = as_bf16x8(*(const u32x4 *)(pb + (16 * mt + n16) * kPRowBytes + 16 * g));
        shortx8 vb[kPvTiles];
#pragma unroll
        for (int nt = 0; nt < kPvTiles; nt++) {
            const shortx4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p0 + 32 * nt));
            const shortx4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p1 + 32 * nt));
            vb[nt] = shortx8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < kPvTiles; nt++) {
#pragma unroll
            for (int mt = 0; mt < kHt; mt++) // head tiles past the group's heads see P = 0
                o[mt][nt] = mfma16x16x32(__builtin_bit_cast(bf16x8, vb[nt]), pa[mt], o[mt][nt]);
        }
    };

    __syncthreads(); // rowidx, resc cleared
    // Gathers run kDepth steps ahead: buffer j % kDepth holds step j's rows
    // from the step that issues its loads until the step that stages it.
    // Step 0 is staged before the scoring waves start and step 1 while they
    // score it; step i + 2 is staged during step i, and its buffer then
    // takes the loads of step i + 2 + kDepth.
    // Prologue gathers are issued whatever the chunk's step count (a step
    // past the chunk reads latent row 0 and is never staged). With 16- and
    // 32-head groups the step loop is unrolled (at most kMaxSteps steps), so
    // every buffer index is a constant and the loads outstanding at each
    // stage are the same on every path: the compiler's wait before a stage
    // then covers exactly that step's loads, not the later steps' still in
    // flight (measured at 8 x 131072: a workgroup's span from 14.4 to 12.4 us).
    u32x4 rbuf[kDepth][4];
#pragma unroll
    for (int j = 0; j < kDepth; j++)
        gather(rbuf[j], j);
    __builtin_amdgcn_sched_barrier(0); // every prologue load issued before the first wait
    stage(rbuf[0], 0);
    __syncthreads(); // tile 0 staged
    gather(rbuf[0], kDepth);
    if (nsteps > 1)
        stage(rbuf[1], 1);
    gather(rbuf[1 % kDepth], kDepth + 1);
    __syncthreads(); // P of step 0, tile 1 staged
    // step i: PV of step i and staging of step i + 2, while the scoring
    // waves score step i + 1
    if constexpr (G == 64) {
        // A rolled loop (unrolled, the 64-head accumulators and the rows in
        // flight need more registers than a wave has): the buffer of a step
        // is picked at run time, and a gather is issued only for a step the
        // chunk has.
        for (int i = 0; i < nsteps; i++) {
            if (i + 2 < nsteps) {
#pragma unroll
                for (int b = 0; b < kDepth; b++) {
                    if (b == (i + 2) % kDepth) {
                        stage(rbuf[b], i + 2);
                        if (i + 2 + kDepth < nsteps)
                            gather(rbuf[b], i + 2 + kDepth);
                    }
                }
            }
            pv(i);
            __syncthreads();
        }
    } else {
#pragma unroll
        for (int i = 0; i < kMaxSteps; i++) {
            if (i >= nsteps)
                break;
            if (i + 2 < nsteps)
                stage(rbuf[(i + 2) % kDepth], i + 2);
            // steps past kMaxSteps are dropped at compile time; one past the
            // chunk's last step is a wasted read of latent row 0
            if (i + 2 + kDepth < kMaxSteps)
                gather(rbuf[(i + 2) % kDepth], i + 2 + kDepth);
            pv(i);
            __syncthreads();
        }
    }
    __syncthreads(); // mlds

    // Output through LDS: each wave parks its O block (G heads x its 128
    // columns, bf16) in its own region of the now idle tiles, then writes it
    // back as whole 256-byte head rows with 16-byte stores. Only this wave
    // touches its region, so a wait for its own LDS writes is enough.
    constexpr int kORowBytes = 2 * kPvCols + 16; // padded: 16 rows at one column spread over the banks
    static_assert(4 * G * kORowBytes <= (int)sizeof(tile), "O blocks fit the tiles");
    uint8_t *oreg = (uint8_t *)tile + v * (G * kORowBytes);
    const int64_t pbase = (((int64_t)r * hg_count + hg) * nch_max + c) * G;
    auto park = [&](auto scale_of) {
#pragma unroll
        for (int mt = 0; mt < kHt; mt++) {
            const int hl = 16 * mt + n16;
            const float sc = scale_of(hl);
#pragma unroll
            for (int nt = 0; nt < kPvTiles; nt++) {
                u32x2 pk;
                pk.x = pack_bf16x2(o[mt][nt][0] * sc, o[mt][nt][1] * sc);
                pk.y = pack_bf16x2(o[mt][nt][2] * sc, o[mt][nt][3] * sc);
                *(u32x2 *)(oreg + hl * kORowBytes + 2 * (16 * nt + 4 * g)) = pk;
            }
        }
    };
    if (nch == 1) { // the final output: O / l, with kv_scale
        park([&](int hl) {
            const float lh = mlds[hl].y;
            return lh > 0.0f ? kv_scale / lh : 0.0f;
        });
    } else {        // a partial: O as accumulated
        park([](int) { return 1.0f; });
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane: 16 bytes (8 columns) of head row 4 i + (lane >> 4)
    const int cb = 16 * (lane & 15);
#pragma unroll
    for (int i = 0; i < G / 4; i++) {
        const int hl = 4 * i + (lane >> 4);
        const int h = h0 + hl;
        const u32x4 val = *(const u32x4 *)(oreg + hl * kORowBytes + cb);
        if (hl < nh) {
            uint16_t *orow = (nch == 1) ? out + ((int64_t)r * H + h) * kLat
                                        : part_o + (pbase + hl) * kLat;
            // streaming store: the partials are read once, by the merge
            // (measured: -1 us per step at 8 x 131072 and 64 x 16.4k)
            __builtin_nontemporal_store(val, (u32x4 *)((uint8_t *)(orow + kPvCols * v) + cb));
        }
    }
}

// Fold the per-chunk partials of every (row, head) in chunk order.
// (the partial pointers carry no __restrict__, so the first batch's loads are
// not sunk below the row-length test: loads through const restrict pointers
// count as invariant and move freely)
__global__ __launch_bounds__(128) void k_mla_merge(const uint16_t *part_o,
                                                   const float2 *part_ml,
                                                   const int32_t *__restrict__ seq_lens,
                                                   uint16_t *__restrict__ out, int H, int top_k,
                                                   int max_len, int nch_max, int hg_count,
                                                   int G, float kv_scale)
{
    const int r = blockIdx.y;
    const int h = blockIdx.x;
    const int hg = h / G;
    const int hl = h % G;
    const int d = threadIdx.x * 4;
    const int64_t pbase = ((int64_t)r * hg_count + hg) * nch_max * G + hl;
    // partials are loaded in unrolled batches (independent loads in flight),
    // then folded strictly in chunk order; straight-line code with selects,
    // so the batch stays in registers. A batch is the chunk count of a row
    // at top_k = 2048 (8 x 256 slots): a larger one re-reads the last chunk
    // (measured: 16 cost 3.5 us per step at 64 x 16.4k)
    constexpr int kB = 8;
    float2 ml[kB];
    floatx4 ov[kB];
    // branch-free: chunks past the last re-read it (and are not folded)
    auto load_batch = [&](int c0, int last) {
#pragma unroll
        for (int k = 0; k < kB; k++) {
            const int64_t pi = pbase + (int64_t)min(c0 + k, last) * G;
            ml[k] = part_ml[pi];
            const u32x2 pk = *(const u32x2 *)(part_o + pi * kLat + d);
            ov[k] = floatx4{__uint_as_float(pk.x << 16), __uint_as_float(pk.x & 0xFFFF0000u),
                            __uint_as_float(pk.y << 16), __uint_as_float(pk.y & 0xFFFF0000u)};
        }
    };
    // the first batch goes out before the row's chunk count is known (every
    // chunk up to nch_max has its place in the workspace)
    load_batch(0, nch_max - 1);
    __asm__ volatile("" ::: "memory"); // those loads stay ahead of the length load and test
    const int L = min(max(seq_lens[r], 0), max_len);
    const int n = min(top_k, L);
    const int nch = (n + kAttChunk - 1) / kAttChunk;
    if (nch <= 1)
        return;
    float m_acc = kNegInf, l_acc = 0.0f;
    floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int c0 = 0; c0 < nch; c0 += kB) {
        if (c0 > 0)
            load_batch(c0, nch - 1);
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
                      const Workspace &wl, hipStream_t stream)
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
    const dim3 grid(nch_max * hgc, ls.num_rows);
    auto kern = G == 16 ? k_mla_decode<16> : G == 32 ? k_mla_decode<32> : k_mla_decode<kAttHeads>;
    hipLaunchKernelGGL(kern, grid, dim3(kAttThreads), 0, stream, q, kv_cache, block_tables,
                       seq_lens, sel, part_o, part_ml, out, ls.rows_per_seq, ls.num_heads,
                       ls.top_k, ls.page_size, ls.max_blocks, ls.num_pages, ls.max_len, kv_scale,
                       qk_log2, nch_max, hgc);
    if (hipGetLastError() != hipSuccess)
        return -1;
    if (nch_max > 1) {
        hipLaunchKernelGGL(k_mla_merge, dim3(ls.num_heads, ls.num_rows), dim3(128), 0, stream,
                           part_o, part_ml, seq_lens, out, ls.num_heads, ls.top_k, ls.max_len,
                           nch_max, hgc, G, kv_scale);
        if (hipGetLastError() != hipSuccess)
            return -1;
    }
    return 0;
}

} // namespace dsa
