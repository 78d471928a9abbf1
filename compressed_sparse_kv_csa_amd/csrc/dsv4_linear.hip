// dsv4_linear.hip -- the projections around the attention core, for gfx950.
//
// HF DeepSeek-V4 page, "Hybrid attention": kv_proj produces the single K=V
// head; the output goes through a grouped low-rank projection (o_groups head
// groups, each to o_lora_rank, then o_b_proj to hidden_size); llm-atlas
// config: hidden_size 4096, q_lora_rank 1024, o_groups 8, o_lora_rank 1024.
// Every one of them is Y = X W^T with both operands K-contiguous (weights
// stored [out, in]); the grouped projection is G such products side by side.
//
// k_linear_big (M and N of at least 1024): 256 x 256 output tiles, K in steps
// of 64, eight waves (4 x 2) each owning 64 x 128 as 4 x 8
// v_mfma_f32_16x16x32_bf16 tiles (fp32 accumulators in VGPRs), so every A
// fragment read from LDS feeds 8 products and every B fragment 4; one
// workgroup of 8 waves per CU (147 KB of LDS).  k_linear (smaller products):
// 128 x 128 tiles, four waves of 4 x 4 tiles, two workgroups per CU.  Both
// load the next K step's operands into registers while the current one is on
// the matrix cores, then write them to the other LDS buffer (rows padded to 72
// elements: the 16 rows one fragment read touches fall in distinct banks).
// Rows past M or N are clamped on load and masked on store.
#include "dsv4_common.h"

namespace dsv4 {

constexpr int kLBM = 128, kLBN = 128, kLBK = 64, kLP = kLBK + 8;

struct LinArgs {
  const uint16_t *x, *w;
  void *y;
  int M, N, K;
  int64_t ldx, ldw, ldy;
  int64_t gx, gw, gy;   // group strides (elements)
};

template <int OUT>
__device__ __forceinline__ void lin_store(void *y, int64_t i, float v) {
  if constexpr (OUT == DSV4_F32) reinterpret_cast<float *>(y)[i] = v;
  else if constexpr (OUT == DSV4_BF16) reinterpret_cast<uint16_t *>(y)[i] = f32_to_bf16(v);
  else {
    const _Float16 h = (_Float16)v;
    __builtin_memcpy(reinterpret_cast<uint16_t *>(y) + i, &h, 2);
  }
}

// grid (ceil(N/128), ceil(M/128), groups), block 256
template <int OUT>
__global__ __launch_bounds__(256, 2) void k_linear(LinArgs L) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kLBM * kLP];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kLBN * kLP];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int wm = wv >> 1, wn = wv & 1;
  const int m0 = blockIdx.y * kLBM, n0 = blockIdx.x * kLBN;
  const uint16_t *X = L.x + (int64_t)blockIdx.z * L.gx;
  const uint16_t *W = L.w + (int64_t)blockIdx.z * L.gw;
  // staging: thread moves 16-byte chunks q = tid + 256 i (i < 4) of each
  // 128 x 64 operand tile: row q / 8, k chunk q % 8
  u32x4 sa[4], sb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, row = q >> 3, kc = q & 7;
      const int m = min(m0 + row, L.M - 1), n = min(n0 + row, L.N - 1);
      sa[i] = *reinterpret_cast<const u32x4 *>(X + (int64_t)m * L.ldx + k0 + 8 * kc);
      sb[i] = *reinterpret_cast<const u32x4 *>(W + (int64_t)n * L.ldw + k0 + 8 * kc);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, row = q >> 3, kc = q & 7;
      *reinterpret_cast<u32x4 *>(&As[buf][row * kLP + 8 * kc]) = sa[i];
      *reinterpret_cast<u32x4 *>(&Bs[buf][row * kLP + 8 * kc]) = sb[i];
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = L.K / kLBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load((kt + 1) * kLBK);   // in flight during this step's MFMAs
#pragma unroll
    for (int kk = 0; kk < kLBK; kk += 32) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(&As[buf][(64 * wm + 16 * i + c) * kLP + kk + 8 * g]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8 *>(&Bs[buf][(64 * wn + 16 * j + c) * kLP + kk + 8 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store(buf ^ 1);
    __syncthreads();
  }
  // lane (c, g) of tile (i, j) holds rows 16i + 4g + v, column 16j + c
  void *Y = L.y;
  const int64_t ybase = (int64_t)blockIdx.z * L.gy;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 64 * wn + 16 * j + c;
      if (n >= L.N) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 64 * wm + 16 * i + 4 * g + v;
        if (m < L.M) lin_store<OUT>(Y, ybase + (int64_t)m * L.ldy + n, acc[i][j][v]);
      }
    }
}

constexpr int kBBM = 256, kBBN = 256, kBBK = 64, kBP = kBBK + 8;
template <int OUT>
__global__ __launch_bounds__(512, 1) void k_linear_big(LinArgs L) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBBM * kBP];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBBN * kBP];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int wm = wv >> 1, wn = wv & 1;
  const int m0 = blockIdx.y * kBBM, n0 = blockIdx.x * kBBN;
  const uint16_t *X = L.x + (int64_t)blockIdx.z * L.gx;
  const uint16_t *W = L.w + (int64_t)blockIdx.z * L.gw;
  u32x4 sa[4], sb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 512 * i, row = q >> 3, kc = q & 7;
      const int m = min(m0 + row, L.M - 1), n = min(n0 + row, L.N - 1);
      sa[i] = *reinterpret_cast<const u32x4 *>(X + (int64_t)m * L.ldx + k0 + 8 * kc);
      sb[i] = *reinterpret_cast<const u32x4 *>(W + (int64_t)n * L.ldw + k0 + 8 * kc);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 512 * i, row = q >> 3, kc = q & 7;
      *reinterpret_cast<u32x4 *>(&As[buf][row * kBP + 8 * kc]) = sa[i];
      *reinterpret_cast<u32x4 *>(&Bs[buf][row * kBP + 8 * kc]) = sb[i];
    }
  };
  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int KT = L.K / kBBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load((kt + 1) * kBBK);
#pragma unroll
    for (int kk = 0; kk < kBBK; kk += 32) {
      bf16x8 a[4], b[8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(&As[buf][(64 * wm + 16 * i + c) * kBP + kk + 8 * g]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        b[j] = *reinterpret_cast<const bf16x8 *>(&Bs[buf][(128 * wn + 16 * j + c) * kBP + kk + 8 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store(buf ^ 1);
    __syncthreads();
  }
  void *Y = L.y;
  const int64_t ybase = (int64_t)blockIdx.z * L.gy;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = n0 + 128 * wn + 16 * j + c;
      if (n >= L.N) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 64 * wm + 16 * i + 4 * g + v;
        if (m < L.M) lin_store<OUT>(Y, ybase + (int64_t)m * L.ldy + n, acc[i][j][v]);
      }
    }
}

}  // namespace dsv4

using namespace dsv4;

namespace dsv4host {

int launch_linear(const void *x, int64_t ldx, const void *w, int64_t ldw, void *y, int64_t ldy, int y_dtype, int M,
                  int N, int K, int groups, int64_t gx, int64_t gw, int64_t gy, hipStream_t st) {
  if (M == 0 || N == 0 || groups == 0) return DSV4_OK;
  LinArgs L{(const uint16_t *)x, (const uint16_t *)w, y, M, N, K, ldx, ldw, ldy, gx, gw, gy};
  if (M >= 1024 && N >= 1024) {
    dim3 g2((unsigned)((N + kBBN - 1) / kBBN), (unsigned)((M + kBBM - 1) / kBBM), (unsigned)groups), b2(512);
    if (y_dtype == DSV4_F32) hipLaunchKernelGGL(k_linear_big<DSV4_F32>, g2, b2, 0, st, L);
    else if (y_dtype == DSV4_BF16) hipLaunchKernelGGL(k_linear_big<DSV4_BF16>, g2, b2, 0, st, L);
    else hipLaunchKernelGGL(k_linear_big<DSV4_F16>, g2, b2, 0, st, L);
    return check_launch("k_linear_big");
  }
  dim3 grid((unsigned)((N + kLBN - 1) / kLBN), (unsigned)((M + kLBM - 1) / kLBM), (unsigned)groups), block(256);
  if (y_dtype == DSV4_F32) hipLaunchKernelGGL(k_linear<DSV4_F32>, grid, block, 0, st, L);
  else if (y_dtype == DSV4_BF16) hipLaunchKernelGGL(k_linear<DSV4_BF16>, grid, block, 0, st, L);
  else hipLaunchKernelGGL(k_linear<DSV4_F16>, grid, block, 0, st, L);
  return check_launch("k_linear");
}

}  // namespace dsv4host
