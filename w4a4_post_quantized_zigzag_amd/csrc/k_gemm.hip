// W4A4 GEMM: packed int4 activations [M][K/2] x packed int4 weights [N][K/2] -> int32 on int8 MFMA,
// with the dequantization (per-token or per-step activation scale, per-output-channel weight
// scale), optional GELU / residual epilogue and the fp16 store fused into the tile's epilogue.
//
// CDNA4 has no int4 matrix instruction and its FP4 format (e2m1) does not hold the uniform int4
// grid, so nibbles are widened to int8 while being staged into LDS and fed to
// v_mfma_i32_16x16x64_i8. The widening keeps each nibble in the high half of its byte,
// (v << 4) & 0xF0F0F0F0 for the even codes and v & 0xF0F0F0F0 for the odd ones, so every int8
// operand equals 16 * code exactly and the MFMA sums 256 * q * p; an arithmetic shift right by 8
// recovers the exact integer sum (|sum| <= 64 K, so 256 * 64 K stays below 2^31 for the at most
// 2^16 k values of one split). Both operands go through the same even/odd reordering of k, so the dot products match.
#include "w4a4_internal.h"

namespace w4a4 {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int KS = 64;        // k elements per pipeline step
constexpr int KSB = KS / 2;   // packed bytes per row per step
constexpr int LDS_ROW = 80;   // bytes per staged int8 row (64 + 16 pad against bank conflicts)
constexpr int MAX_K_SPLIT = 1 << 16;  // 256 * 64 * 2^16 = 2^30 fits int32

__device__ __forceinline__ void widen16(const uint4 &p, uint4 &lo, uint4 &hi)
{
    // 16 packed bytes (k = 0..31 of a half step) -> 32 int8 values, two dwords per packed dword
    lo.x = (p.x << 4) & 0xF0F0F0F0u; lo.y = p.x & 0xF0F0F0F0u;
    lo.z = (p.y << 4) & 0xF0F0F0F0u; lo.w = p.y & 0xF0F0F0F0u;
    hi.x = (p.z << 4) & 0xF0F0F0F0u; hi.y = p.z & 0xF0F0F0F0u;
    hi.z = (p.w << 4) & 0xF0F0F0F0u; hi.w = p.w & 0xF0F0F0F0u;
}

// Load 16 packed bytes of row `row` at packed byte offset `kb`; zero outside [0, rows) x [0, kbend).
template <bool VEC>
__device__ __forceinline__ uint4 load_packed16(const uint8_t *__restrict__ base, int rows, int row,
                                               int64_t ld, int kb, int kbend)
{
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row >= rows) return v;
    const uint8_t *p = base + (int64_t)row * ld + kb;
    if (VEC && kb + 16 <= kbend) {
        v = *reinterpret_cast<const uint4 *>(p);
    } else {
        uint32_t w[4] = {0, 0, 0, 0};
        for (int t = 0; t < 16; ++t)
            if (kb + t < kbend) w[t >> 2] |= (uint32_t)p[t] << (8 * (t & 3));
        v = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return v;
}

__device__ __forceinline__ float gelu_erf(float v)
{
    return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v)
{
    return __half_as_ushort(__float2half_rn(v));
}

// BM x BN output tile, 4 waves as WAVES_M x WAVES_N, each wave (BM/WAVES_M) x (BN/WAVES_N) made of
// 16x16 MFMA fragments. grid = (N tiles, M tiles, k splits).
template <int BM, int BN, int WAVES_M, int WAVES_N, bool VEC>
__global__ __launch_bounds__(256) void k_gemm_w4a4(const uint8_t *__restrict__ xq,
                                                   const uint8_t *__restrict__ wq, int M, int N,
                                                   int K, int k_split, GemmEpilogue epi,
                                                   int32_t *__restrict__ partial)
{
#pragma clang fp contract(off)
    static_assert(WAVES_M * WAVES_N == 4, "4 waves");
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * LDS_ROW];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * LDS_ROW];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int64_t ldp = K / 2;
    const int kb_begin = blockIdx.z * (k_split / 2);
    const int kb_end = min(kb_begin + k_split / 2, (int)ldp);
    const int steps = (kb_end - kb_begin + KSB - 1) / KSB;

    v4i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    // staging assignment: each (row, half) pair is 16 packed bytes
    constexpr int A_ITEMS = BM * 2, B_ITEMS = BN * 2;
    constexpr int A_PER = (A_ITEMS + 255) / 256, B_PER = (B_ITEMS + 255) / 256;
    uint4 ra[A_PER], rb[B_PER];

    auto gload = [&](int step) {
        const int kb = kb_begin + step * KSB;
#pragma unroll
        for (int t = 0; t < A_PER; ++t) {
            int item = tid + t * 256;
            ra[t] = make_uint4(0, 0, 0, 0);
            if (item < A_ITEMS)
                ra[t] = load_packed16<VEC>(xq, M, m0 + (item >> 1), ldp, kb + 16 * (item & 1),
                                           kb_end);
        }
#pragma unroll
        for (int t = 0; t < B_PER; ++t) {
            int item = tid + t * 256;
            rb[t] = make_uint4(0, 0, 0, 0);
            if (item < B_ITEMS)
                rb[t] = load_packed16<VEC>(wq, N, n0 + (item >> 1), ldp, kb + 16 * (item & 1),
                                           kb_end);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int t = 0; t < A_PER; ++t) {
            int item = tid + t * 256;
            if (item < A_ITEMS) {
                uint4 lo, hi;
                widen16(ra[t], lo, hi);
                uint8_t *dst = &sA[buf][(item >> 1) * LDS_ROW + 32 * (item & 1)];
                *reinterpret_cast<uint4 *>(dst) = lo;
                *reinterpret_cast<uint4 *>(dst + 16) = hi;
            }
        }
#pragma unroll
        for (int t = 0; t < B_PER; ++t) {
            int item = tid + t * 256;
            if (item < B_ITEMS) {
                uint4 lo, hi;
                widen16(rb[t], lo, hi);
                uint8_t *dst = &sB[buf][(item >> 1) * LDS_ROW + 32 * (item & 1)];
                *reinterpret_cast<uint4 *>(dst) = lo;
                *reinterpret_cast<uint4 *>(dst + 16) = hi;
            }
        }
    };

    if (steps > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();
    const int frow = lane & 15, fk = (lane >> 4) * 16;
    for (int st = 0; st < steps; ++st) {
        const int buf = st & 1;
        if (st + 1 < steps) gload(st + 1);
        v4i a[FM], b[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            a[i] = *reinterpret_cast<const v4i *>(&sA[buf][(wm * WTM + i * 16 + frow) * LDS_ROW + fk]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            b[j] = *reinterpret_cast<const v4i *>(&sB[buf][(wn * WTN + j * 16 + frow) * LDS_ROW + fk]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        if (st + 1 < steps) lstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: fragment (i, j) register r holds row 4*(lane/16) + r, column lane % 16
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * WTN + j * 16 + (lane & 15);
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * WTM + i * 16 + 4 * (lane >> 4) + r;
                if (m >= M) continue;
                const int32_t v = acc[i][j][r] >> 8;
                if (partial) {
                    partial[((int64_t)blockIdx.z * M + m) * N + n] = v;
                    continue;
                }
                if (epi.mode == GEMM_OUT_I32) {
                    epi.acc_out[(int64_t)m * N + n] = v;
                    continue;
                }
                const float sx = epi.x_scale_per_token ? epi.x_scale[m] : epi.x_scale[0];
                float y = (float)v * sx;
                y = y * epi.w_scale[n];
                if (epi.mode == W4A4_EPI_GELU) y = gelu_erf(y);
                else if (epi.mode == W4A4_EPI_RESIDUAL)
                    y = y + __half2float(__ushort_as_half(epi.residual[(int64_t)m * epi.ldr + n]));
                epi.Y[(int64_t)m * epi.ldy + n] = f32_to_f16_bits(y);
            }
        }
    }
}

// Split-K reduction of exact int32 partials, then the same epilogue.
__global__ void k_splitk_epilogue(const int32_t *__restrict__ partial, int splits, int M, int N,
                                  GemmEpilogue epi)
{
#pragma clang fp contract(off)
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)M * N) return;
    const int m = (int)(idx / N), n = (int)(idx % N);
    int32_t v = 0;
    for (int s = 0; s < splits; ++s) v += partial[(int64_t)s * M * N + idx];
    if (epi.mode == GEMM_OUT_I32) {
        epi.acc_out[idx] = v;
        return;
    }
    const float sx = epi.x_scale_per_token ? epi.x_scale[m] : epi.x_scale[0];
    float y = (float)v * sx;
    y = y * epi.w_scale[n];
    if (epi.mode == W4A4_EPI_GELU) y = gelu_erf(y);
    else if (epi.mode == W4A4_EPI_RESIDUAL)
        y = y + __half2float(__ushort_as_half(epi.residual[(int64_t)m * epi.ldr + n]));
    epi.Y[(int64_t)m * epi.ldy + n] = f32_to_f16_bits(y);
}

struct GemmPlan {
    int bm, bn, splits, k_split;
};

static GemmPlan plan_gemm(int M, int N, int K)
{
    GemmPlan p;
    if (M <= 64) {
        p.bm = 64;
        p.bn = 64;
    } else {
        p.bm = 128;
        p.bn = 128;
    }
    const int64_t tiles = (int64_t)((N + p.bn - 1) / p.bn) * ((M + p.bm - 1) / p.bm);
    int splits = 1;
    // long K with too few tiles to fill 256 compute units: split K into exact int32 partials
    while (tiles * splits < 256 && K / (splits * 2) >= 2048) splits *= 2;
    int k_split = (K + splits - 1) / splits;
    k_split = (k_split + KS - 1) / KS * KS;
    while (k_split > MAX_K_SPLIT) {
        splits *= 2;
        k_split = ((K + splits - 1) / splits + KS - 1) / KS * KS;
    }
    splits = (K + k_split - 1) / k_split;
    p.splits = splits;
    p.k_split = k_split;
    return p;
}

size_t gemm_workspace(int M, int N, int K)
{
    GemmPlan p = plan_gemm(M, N, K);
    if (p.splits <= 1) return 0;
    return (size_t)p.splits * (size_t)M * (size_t)N * sizeof(int32_t);
}

template <int BM, int BN, int WM, int WN>
static void launch_tile(bool vec, dim3 grid, hipStream_t s, const uint8_t *xq, const uint8_t *wq,
                        int M, int N, int K, int k_split, const GemmEpilogue &epi, int32_t *partial)
{
    if (vec)
        hipLaunchKernelGGL((k_gemm_w4a4<BM, BN, WM, WN, true>), grid, dim3(256), 0, s, xq, wq, M, N,
                           K, k_split, epi, partial);
    else
        hipLaunchKernelGGL((k_gemm_w4a4<BM, BN, WM, WN, false>), grid, dim3(256), 0, s, xq, wq, M,
                           N, K, k_split, epi, partial);
}

int launch_gemm(const uint8_t *xq, const uint8_t *wq, int M, int N, int K, const GemmEpilogue &epi,
                void *ws, size_t ws_bytes, hipStream_t s)
{
    if (M == 0) return W4A4_OK;
    GemmPlan p = plan_gemm(M, N, K);
    const bool vec = ((K / 2) % 16 == 0) && ((uintptr_t)xq % 16 == 0) && ((uintptr_t)wq % 16 == 0);
    int32_t *partial = nullptr;
    if (p.splits > 1) {
        if (!ws || ws_bytes < gemm_workspace(M, N, K))
            return fail(W4A4_ERR_WORKSPACE, "gemm needs %zu workspace bytes",
                        gemm_workspace(M, N, K));
        partial = reinterpret_cast<int32_t *>(ws);
    }
    dim3 grid((N + p.bn - 1) / p.bn, (M + p.bm - 1) / p.bm, p.splits);
    if (p.bm == 64)
        launch_tile<64, 64, 1, 4>(vec, grid, s, xq, wq, M, N, K, p.k_split, epi, partial);
    else
        launch_tile<128, 128, 2, 2>(vec, grid, s, xq, wq, M, N, K, p.k_split, epi, partial);
    int rc = check_launch("gemm");
    if (rc != W4A4_OK || p.splits <= 1) return rc;
    const int64_t total = (int64_t)M * N;
    hipLaunchKernelGGL(k_splitk_epilogue, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       partial, p.splits, M, N, epi);
    return check_launch("gemm split-k epilogue");
}

}  // namespace w4a4
