// cache_write.hip -- the cache-write side that feeds the decode path: for
// each row, the token at pos = seq_lens[r] - 1 is stored in both caches.
//
//  - latent row: the plain RMSNorm x * rms * w with rms = 1/sqrt(mean(x^2) +
//    eps) (glm5next_dsa/layer.rs source page: module header, first trap --
//    the vanilla form, not 1 + w), scaled by 1/kv_scale (the `kv_scale` field
//    doc: the write takes 1/scale), encoded to OCP E4M3 and written to the
//    paged slot page * page_size + pos % page_size with page =
//    block_table[pos / page_size] (the `latent_write` kernel handle:
//    RMSNorm + FP8 + paged slot write; `decode_k`: the slot arithmetic).
//  - indexer key row: LayerNorm with a bias (module header, second trap),
//    (x - mean) / sqrt(var + eps) * w + b, stored as bf16 at
//    k_normed[s][pos] (`indexer_forward`: the key row lands at the
//    position the indexer cache advances to), and, when the caller keeps
//    them, the position's validity mark valid[s][pos] = 1 with it
//    (`indexer_forward`: placement and the mark both from the device
//    position, never a host-baked address).
//
// One workgroup per row: 256 threads normalise the 512-wide latent (two
// values each), wave 0 also normalises the key row. Sums run in fp32 in a
// fixed order (DPP within a wave, then the four waves in order), so results
// are deterministic. Values beyond +-448 saturate before the E4M3 encode.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kCwThreads = 256;
constexpr int kCwLat = 512;

// Sum of one float per lane over the wave, in every lane (fixed order).
__device__ __forceinline__ float wave_sum_f32(float v)
{
    auto step = [](float x, uint32_t moved) { return x + __uint_as_float(moved); };
    v = step(v, dpp_u32<kDppQuadXor1>(__float_as_uint(v)));
    v = step(v, dpp_u32<kDppQuadXor2>(__float_as_uint(v)));
    v = step(v, dpp_u32<kDppRowHalfMirror>(__float_as_uint(v)));
    v = step(v, dpp_u32<kDppRowMirror>(__float_as_uint(v)));
    const float r0 = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 0));
    const float r1 = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 16));
    const float r2 = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 32));
    const float r3 = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

template <int D>
__global__ __launch_bounds__(kCwThreads) void k_cache_write(
    const uint16_t *__restrict__ kv_a, const uint16_t *__restrict__ latent_w,
    const uint16_t *__restrict__ k_proj, const uint16_t *__restrict__ k_w,
    const uint16_t *__restrict__ k_b, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ bt, uint8_t *__restrict__ kv_cache, uint16_t *__restrict__ k_normed,
    uint8_t *__restrict__ valid, int K, int ps, int max_blocks, int num_pages, int64_t cap,
    int max_len, float eps, float inv_kv_scale)
{
    __shared__ float part[kCwThreads / kWave];
    const int r = blockIdx.x;
    const int s = r / K;
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int L = seq_lens[r];
    if (L < 1 || L > max_len)
        return;
    const int pos = L - 1;

    // ---- latent row: two values per thread ----
    const uint32_t xb = *(const uint32_t *)(kv_a + (int64_t)r * kCwLat + 2 * tid);
    const uint32_t wb = *(const uint32_t *)(latent_w + 2 * tid);
    const float x0 = bf16_bits_to_f32(xb & 0xFFFFu), x1 = bf16_bits_to_f32(xb >> 16);
    const float ws = wave_sum_f32(__builtin_fmaf(x0, x0, x1 * x1));
    if (lane == 0)
        part[wave] = ws;
    __syncthreads();
    const float ss = (part[0] + part[1]) + (part[2] + part[3]);
    const float rms = 1.0f / __builtin_sqrtf(ss / (float)kCwLat + eps);
    const float y0 = x0 * rms * bf16_bits_to_f32(wb & 0xFFFFu) * inv_kv_scale;
    const float y1 = x1 * rms * bf16_bits_to_f32(wb >> 16) * inv_kv_scale;
    const int logical = pos / ps;
    const int page = logical < max_blocks ? bt[(int64_t)s * max_blocks + logical] : -1;
    if (page >= 0 && page < num_pages) {
        const float c0 = __builtin_fminf(__builtin_fmaxf(y0, -448.0f), 448.0f);
        const float c1 = __builtin_fminf(__builtin_fmaxf(y1, -448.0f), 448.0f);
        const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
        uint8_t *dst = kv_cache + ((int64_t)page * ps + pos % ps) * kCwLat + 2 * tid;
        *(uint16_t *)dst = (uint16_t)(packed & 0xFFFF);
    }

    // ---- indexer key row: wave 0, D / 64 values per lane ----
    if (wave == 0 && pos < cap) {
        constexpr int V = D / kWave;
        const uint16_t *kr = k_proj + (int64_t)r * D + V * lane;
        float x[V];
#pragma unroll
        for (int i = 0; i < V; i++)
            x[i] = bf16_bits_to_f32(kr[i]);
        float sx = 0.0f;
#pragma unroll
        for (int i = 0; i < V; i++)
            sx += x[i];
        const float mean = wave_sum_f32(sx) / (float)D;
        float sd = 0.0f;
#pragma unroll
        for (int i = 0; i < V; i++)
            sd = __builtin_fmaf(x[i] - mean, x[i] - mean, sd);
        const float var = wave_sum_f32(sd) / (float)D;
        const float inv = 1.0f / __builtin_sqrtf(var + eps);
        uint16_t *dst = k_normed + ((int64_t)s * cap + pos) * D + V * lane;
#pragma unroll
        for (int i = 0; i < V; i++) {
            const float y = (x[i] - mean) * inv * bf16_bits_to_f32(k_w[V * lane + i]) +
                            bf16_bits_to_f32(k_b[V * lane + i]);
            dst[i] = f32_to_bf16_rne(y);
        }
        if (valid != nullptr && lane == 0)
            valid[(int64_t)s * cap + pos] = 1;
    }
}

int launch_cache_write(const LaunchShape &ls, const uint16_t *kv_a, const uint16_t *latent_w,
                       const uint16_t *k_proj, const uint16_t *k_w, const uint16_t *k_b,
                       const int32_t *seq_lens, const int32_t *block_tables, float eps,
                       float kv_scale, uint8_t *kv_cache, uint16_t *k_normed, uint8_t *valid,
                       hipStream_t stream)
{
    const float inv = (float)(1.0 / (double)kv_scale);
    if (ls.index_dim == 128)
        hipLaunchKernelGGL(k_cache_write<128>, dim3(ls.num_rows), dim3(kCwThreads), 0, stream,
                           kv_a, latent_w, k_proj, k_w, k_b, seq_lens, block_tables, kv_cache,
                           k_normed, valid, ls.rows_per_seq, ls.page_size, ls.max_blocks,
                           ls.num_pages,
                           (int64_t)ls.k_capacity, ls.max_len, eps, inv);
    else if (ls.index_dim == 64)
        hipLaunchKernelGGL(k_cache_write<64>, dim3(ls.num_rows), dim3(kCwThreads), 0, stream,
                           kv_a, latent_w, k_proj, k_w, k_b, seq_lens, block_tables, kv_cache,
                           k_normed, valid, ls.rows_per_seq, ls.page_size, ls.max_blocks,
                           ls.num_pages,
                           (int64_t)ls.k_capacity, ls.max_len, eps, inv);
    else
        return -1;
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

} // namespace dsa
