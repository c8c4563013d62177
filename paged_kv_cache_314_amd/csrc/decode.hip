// Split-KV flash-decode for paged K/V on gfx950 (one query token per sequence).
//
// Operation: aclnnFusedInferAttentionScoreV4, "Function" (softmax(scale*QK^T + mask) V,
// per row), decode scenario (one query token); paged K/V per the paged-attention
// constraints of aclnnFusedInferAttentionScoreV3 (token t of sequence b in block
// blockTables[b][t / blockSize], slot t % blockSize); GQA per its numHeads /
// numKeyValueHeads constraint; int8 K/V with per-channel antiquant scales.
//
// Work decomposition (planned on the host): one workgroup = 4 waves = one
// (sequence, kv head, group of <= 16 query heads, range of 32-token tiles).  Each wave
// streams its own contiguous sub-range of tiles with a private online softmax; the four
// wave states are merged in LDS, then written either as the final out/lse (single
// split) or as an un-normalised partial (m, l, O) that the combine kernel merges in a
// fixed order.
//
// Per 32-token tile a wave does, for its 16 packed query heads:
//   S[16 tok x 16 heads] = K_tile . Q^T        2 x (headSize/32) MFMA 16x16x32
//   online softmax on S (in registers; 2 cross-lane steps per reduction)
//   O^T[16 d x 16 heads] += V^T . P^T          8 MFMA 16x16x32 (one per d-phase)
// K rows are MFMA A-operands straight from global memory (each lane reads 16 contiguous
// bytes of one token row).  V is read as 8 token rows x 16 bytes per lane, four whole
// rows per load instruction, and transposed in registers (8x8 of 16-bit values), so no
// LDS traffic is needed on the streaming path.  Tokens are visited in the permuted
// order that makes the S accumulator layout equal the P^T operand layout.
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_kernels.h"

namespace pa {

namespace {

// d-chunk (in units of 8 elements) that lane group qg covers at QK k-step kk.
// 16-bit K rows: chunk 4*kk + qg (a load instruction covers 64 contiguous bytes per row).
// int8 K rows: each lane loads 16 bytes = 2 chunks, chunks 2*(qg + 4*(kk/2)) + kk%2.
template <bool I8>
__device__ __forceinline__ int dchunk(int qg, int kk) {
    if constexpr (I8) return 2 * (qg + 4 * (kk >> 1)) + (kk & 1);
    else return 4 * kk + qg;
}

template <int D, bool BF16, bool I8>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a) {
    constexpr int KK = D / 32;                 // QK k-steps
    constexpr int KP = D / 64;                 // int8 16-byte loads per K row
    constexpr bool MBF = BF16 && !I8;          // MFMA element type (int8 path runs in f16)
    constexpr int VCOLS = D / 8;               // lanes (per row) that hold V columns

    __shared__ float s_m[kDecodeWaves][kHeadPack];
    __shared__ float s_l[kDecodeWaves][kHeadPack];
    __shared__ float s_o[kDecodeWaves][kHeadPack][D];

    const DecodeItem it = a.items[blockIdx.x];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;                 // packed head (QK/PV column)
    const int qg = lane >> 4;                  // lane group: k-slots 8*qg .. 8*qg+7
    const int hl = it.hg * kHeadPack + col;    // head index within the kv group
    const bool hvalid = hl < a.group;
    const int head = it.kvh * a.group + (hvalid ? hl : 0);
    const int kvlen = it.kvlen;

    // ------------------------------------------------------------ Q operand
    u32x4 qhi[KK], qlo[KK];
    float s_mul;                               // multiplies the raw MFMA score
    if constexpr (!I8) {
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                               static_cast<int64_t>(it.qrow) * a.q_tok_stride +
                               static_cast<int64_t>(head) * a.q_head_stride;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qhi[kk] = hvalid ? *reinterpret_cast<const u32x4*>(qrow + 8 * dchunk<I8>(qg, kk)) : z;
            qlo[kk] = z;
        }
        s_mul = a.scale_log2;
    } else {
        // q' = q * sK * qkScale * log2(e), brought to |q'| < 2^14 by a power of two and
        // split into f16 hi + lo, so that the f16 MFMA sees q' to ~22 bits.
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                               static_cast<int64_t>(it.qrow) * a.q_tok_stride +
                               static_cast<int64_t>(head) * a.q_head_stride;
        float qf[KK][8];
        float amax = 0.0f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int d0 = 8 * dchunk<I8>(qg, kk);
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (hvalid) raw = *reinterpret_cast<const u32x4*>(qrow + d0);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t w = raw[e >> 1];
                const float qv = half_to_f32<BF16>((e & 1) ? (w >> 16) : (w & 0xffffu));
                const int d = d0 + e;
                float sk;
                if (a.scale_is_f32) {
                    sk = static_cast<const float*>(a.kscale)[it.kvh * D + d];
                } else {
                    sk = half_to_f32<BF16>(static_cast<const uint16_t*>(a.kscale)[it.kvh * D + d]);
                }
                qf[kk][e] = qv * sk * a.scale_log2;
                amax = fmaxf(amax, fabsf(qf[kk][e]));
            }
        }
        amax = fmaxf(amax, shfl_xor_f(amax, 16));
        amax = fmaxf(amax, shfl_xor_f(amax, 32));
        int ex = 0;
        if (amax > 0.0f && amax < INFINITY) {
            int x;
            frexpf(amax, &x);                  // amax = f * 2^x, f in [0.5, 1)
            ex = 14 - x;
            ex = ex > 120 ? 120 : (ex < -120 ? -120 : ex);
        }
        const float up = ldexpf(1.0f, ex);
        s_mul = ldexpf(1.0f, -ex);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float x0 = qf[kk][e] * up, x1 = qf[kk][e + 1] * up;
                const _Float16 h0 = static_cast<_Float16>(x0), h1 = static_cast<_Float16>(x1);
                const _Float16 l0 = static_cast<_Float16>(x0 - static_cast<float>(h0));
                const _Float16 l1 = static_cast<_Float16>(x1 - static_cast<float>(h1));
                qhi[kk][e >> 1] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h0)) |
                                  (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
                qlo[kk][e >> 1] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l0)) |
                                  (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l1)) << 16);
            }
        }
    }
    float slope2 = 0.0f;
    if (a.mask_type == PA_MASK_ALIBI) slope2 = a.slopes[head] * kLog2e;
    const int pos = kvlen - 1;                  // absolute position of the decode query

    // --------------------------------------------------------------- state
    float m_run = -INFINITY;                    // running max (log2 units) of head `col`
    float l_run = 0.0f;                         // this lane's share of the running sum
    f32x4 acc[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ntiles = it.t1 - it.t0;
    const int w0 = it.t0 + (ntiles * wave) / kDecodeWaves;
    const int w1 = it.t0 + (ntiles * (wave + 1)) / kDecodeWaves;
    const int32_t* trow = a.table + static_cast<int64_t>(it.b) * a.table_stride;
    const int bs = a.block_size;
    const int64_t k_head_off = static_cast<int64_t>(it.kvh) * a.k_head_stride;
    const int64_t v_head_off = static_cast<int64_t>(it.kvh) * a.v_head_stride;

    for (int tile = w0; tile < w1; ++tile) {
        const int T = tile * kDecodeTile;
        // Blocks holding tokens T .. T+31: at most three (blockSize >= 16).
        const int blk_a = T / bs;
        const int r0 = T - blk_a * bs;
        const int e0 = trow[blk_a];
        const int e1 = ((blk_a + 1) * bs < kvlen) ? trow[blk_a + 1] : 0;
        const int e2 = ((blk_a + 2) * bs < kvlen) ? trow[blk_a + 2] : 0;
        auto token_addr = [&](int delta, int64_t blk_stride, int64_t slot_stride,
                              int64_t head_off) -> int64_t {
            int u = r0 + delta;
            int nb = (u >= bs) + (u >= 2 * bs);
            int phys = nb == 0 ? e0 : (nb == 1 ? e1 : e2);
            return static_cast<int64_t>(phys) * blk_stride +
                   static_cast<int64_t>(u - nb * bs) * slot_stride + head_off;
        };

        // ---- K tile (MFMA A operand: lane row = token T + 16m + col)
        u32x4 kop[2][KK];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int delta = 16 * m + col;
            const bool ok = T + delta < kvlen;
            const int64_t off = ok ? token_addr(delta, a.k_blk_stride, a.k_slot_stride, k_head_off) : 0;
            if constexpr (!I8) {
                const uint16_t* krow = static_cast<const uint16_t*>(a.k) + off;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    u32x4 z = {0u, 0u, 0u, 0u};
                    kop[m][kk] = ok ? *reinterpret_cast<const u32x4*>(krow + 8 * dchunk<I8>(qg, kk)) : z;
                }
            } else {
                const int8_t* krow = static_cast<const int8_t*>(a.k) + off;
#pragma unroll
                for (int kp = 0; kp < KP; ++kp) {
                    u32x4 raw = {0u, 0u, 0u, 0u};
                    if (ok) raw = *reinterpret_cast<const u32x4*>(krow + 16 * (qg + 4 * kp));
                    // 16 int8 -> two k-steps of 8 f16 each
                    const u32x2 c0 = i8x4_to_f16x4(raw.x), c1 = i8x4_to_f16x4(raw.y);
                    const u32x2 c2 = i8x4_to_f16x4(raw.z), c3 = i8x4_to_f16x4(raw.w);
                    kop[m][2 * kp] = u32x4{c0.x, c0.y, c1.x, c1.y};
                    kop[m][2 * kp + 1] = u32x4{c2.x, c2.y, c3.x, c3.y};
                }
            }
        }
        // ---- V tile rows: token T + 16*(r/4) + 4*qg + r%4, columns 8*col .. 8*col+7
        u32x4 vrow[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int delta = 16 * (r >> 2) + 4 * qg + (r & 3);
            const bool ok = (T + delta < kvlen) && (col < VCOLS);
            const int64_t off = ok ? token_addr(delta, a.v_blk_stride, a.v_slot_stride, v_head_off) : 0;
            u32x4 z = {0u, 0u, 0u, 0u};
            if constexpr (!I8) {
                const uint16_t* vp = static_cast<const uint16_t*>(a.v) + off + 8 * col;
                vrow[r] = ok ? *reinterpret_cast<const u32x4*>(vp) : z;
            } else {
                const int8_t* vp = static_cast<const int8_t*>(a.v) + off + 8 * col;
                u32x2 raw = {0u, 0u};
                if (ok) raw = *reinterpret_cast<const u32x2*>(vp);
                const u32x2 c0 = i8x4_to_f16x4(raw.x), c1 = i8x4_to_f16x4(raw.y);
                vrow[r] = ok ? u32x4{c0.x, c0.y, c1.x, c1.y} : z;
            }
        }

        // ---- S = K Q^T, scaled to log2 units, bias + mask
        float s[8];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                c = mfma16x16x32<MBF>(kop[m][kk], qhi[kk], c);
                if constexpr (I8) c = mfma16x16x32<false>(kop[m][kk], qlo[kk], c);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = T + 16 * m + 4 * qg + r;
                float x = c[r] * s_mul;
                if (a.mask_type == PA_MASK_ALIBI) x += slope2 * static_cast<float>(j - pos);
                s[4 * m + r] = (j < kvlen) ? x : -INFINITY;
            }
        }
        // ---- online softmax (head `col`; its 32 scores live in 4 lanes x 8)
        float tmax = s[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, s[i]);
        tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
        tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float p[8];
        float psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = fast_exp2(s[i] - m_use);
            psum += p[i];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[n] *= alpha;
        u32x4 pop;
        pop.x = pack2<MBF>(p[0], p[1]);
        pop.y = pack2<MBF>(p[2], p[3]);
        pop.z = pack2<MBF>(p[4], p[5]);
        pop.w = pack2<MBF>(p[6], p[7]);

        // ---- O^T += V^T P^T: operand n holds column d = 8*col + n of the 8 rows
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            u32x4 vop;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t x = vrow[2 * i][n >> 1], y = vrow[2 * i + 1][n >> 1];
                vop[i] = (n & 1) ? pack_hi(x, y) : pack_lo(x, y);
            }
            acc[n] = mfma16x16x32<MBF>(vop, pop, acc[n]);
        }
    }

    // ------------------------------------------------ merge the 4 wave states
    float l_tot = l_run;
    l_tot += shfl_xor_f(l_tot, 16);
    l_tot += shfl_xor_f(l_tot, 32);
    if (qg == 0) {
        s_m[wave][col] = m_run;
        s_l[wave][col] = l_tot;
    }
    // acc[n][r] = O[head col][d = 32*qg + 8*r + n]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const int d = 32 * qg + 8 * r + n;
            if (d < D) s_o[wave][col][d] = acc[n][r];
        }
    }
    __syncthreads();

    const int geff = a.group < kHeadPack ? a.group : kHeadPack;
    for (int e = threadIdx.x; e < geff * D; e += blockDim.x) {
        const int h = e / D, d = e - (e / D) * D;
        const int hlocal = it.hg * kHeadPack + h;
        if (hlocal >= a.group) continue;
        float M = s_m[0][h];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, s_m[w][h]);
        float L = 0.0f, O = 0.0f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kDecodeWaves; ++w) {
                const float f = fast_exp2(s_m[w][h] - M);
                L += s_l[w][h] * f;
                O += s_o[w][h][d] * f;
            }
        }
        if constexpr (I8) {
            float sv;
            if (a.scale_is_f32) sv = static_cast<const float*>(a.vscale)[it.kvh * D + d];
            else sv = half_to_f32<BF16>(static_cast<const uint16_t*>(a.vscale)[it.kvh * D + d]);
            O *= sv;
        }
        const int out_head = it.kvh * a.group + hlocal;
        if (it.slot < 0) {
            const float val = (L > 0.0f) ? O / L : 0.0f;
            uint16_t* orow = static_cast<uint16_t*>(a.out) +
                             static_cast<int64_t>(it.qrow) * a.out_tok_stride +
                             static_cast<int64_t>(out_head) * a.out_head_stride;
            orow[d] = static_cast<uint16_t>(f32_to_half<BF16>(val));
            if (d == 0 && a.lse != nullptr) {
                a.lse[static_cast<int64_t>(it.qrow) * a.lse_tok_stride + out_head] =
                    (L > 0.0f) ? (M + fast_log2(L)) * kLn2 : INFINITY;
            }
        } else {
            const int64_t sl = static_cast<int64_t>(it.slot) * geff + h;
            a.part_o[sl * D + d] = O;
            if (d == 0) {
                a.part_ml[2 * sl] = M;
                a.part_ml[2 * sl + 1] = L;
            }
        }
    }
}

// Merge the nsplit partials of one (sequence, kv head, head group) in slot order.
template <int D, bool BF16>
__global__ void __launch_bounds__(256) combine_kernel(CombineArgs a) {
    const CombineItem it = a.items[blockIdx.x];
    const int geff = a.group < kHeadPack ? a.group : kHeadPack;
    for (int e = threadIdx.x; e < geff * D; e += blockDim.x) {
        const int h = e / D, d = e - (e / D) * D;
        const int hlocal = it.hg * kHeadPack + h;
        if (hlocal >= a.group) continue;
        float M = -INFINITY;
        for (int s = 0; s < it.nsplit; ++s) {
            const int64_t sl = static_cast<int64_t>(it.slot0 + s) * geff + h;
            M = fmaxf(M, a.part_ml[2 * sl]);
        }
        float L = 0.0f, O = 0.0f;
        if (M != -INFINITY) {
            for (int s = 0; s < it.nsplit; ++s) {
                const int64_t sl = static_cast<int64_t>(it.slot0 + s) * geff + h;
                const float f = fast_exp2(a.part_ml[2 * sl] - M);
                L += a.part_ml[2 * sl + 1] * f;
                O += a.part_o[sl * D + d] * f;
            }
        }
        const int out_head = it.kvh * a.group + hlocal;
        const float val = (L > 0.0f) ? O / L : 0.0f;
        uint16_t* orow = static_cast<uint16_t*>(a.out) +
                         static_cast<int64_t>(it.qrow) * a.out_tok_stride +
                         static_cast<int64_t>(out_head) * a.out_head_stride;
        orow[d] = static_cast<uint16_t>(f32_to_half<BF16>(val));
        if (d == 0 && a.lse != nullptr) {
            a.lse[static_cast<int64_t>(it.qrow) * a.lse_tok_stride + out_head] =
                (L > 0.0f) ? (M + fast_log2(L)) * kLn2 : INFINITY;
        }
    }
}

template <int D, bool BF16, bool I8>
hipError_t launch_decode_t(const DecodeArgs& a, int n_items, hipStream_t stream) {
    hipLaunchKernelGGL((decode_kernel<D, BF16, I8>), dim3(n_items), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_combine_t(const CombineArgs& a, int n_items, hipStream_t stream) {
    hipLaunchKernelGGL((combine_kernel<D, BF16>), dim3(n_items), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int n_items, int head_size, bool bf16, bool i8,
                         hipStream_t stream) {
    if (n_items <= 0) return hipSuccess;
    if (head_size == 128) {
        if (i8) return bf16 ? launch_decode_t<128, true, true>(a, n_items, stream)
                            : launch_decode_t<128, false, true>(a, n_items, stream);
        return bf16 ? launch_decode_t<128, true, false>(a, n_items, stream)
                    : launch_decode_t<128, false, false>(a, n_items, stream);
    }
    if (i8) return bf16 ? launch_decode_t<64, true, true>(a, n_items, stream)
                        : launch_decode_t<64, false, true>(a, n_items, stream);
    return bf16 ? launch_decode_t<64, true, false>(a, n_items, stream)
                : launch_decode_t<64, false, false>(a, n_items, stream);
}

hipError_t launch_combine(const CombineArgs& a, int n_items, int head_size, bool bf16,
                          hipStream_t stream) {
    if (n_items <= 0) return hipSuccess;
    if (head_size == 128)
        return bf16 ? launch_combine_t<128, true>(a, n_items, stream)
                    : launch_combine_t<128, false>(a, n_items, stream);
    return bf16 ? launch_combine_t<64, true>(a, n_items, stream)
                : launch_combine_t<64, false>(a, n_items, stream);
}

}  // namespace pa
