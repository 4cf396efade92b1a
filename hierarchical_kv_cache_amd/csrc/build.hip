// Tree summary builders.
//
// [ZHA] "무엇과 다른가" (how it differs): a chunk's log-mass F(q) = LSE_j(q.k_j/sqrt d)
// is summarised by R tangent planes t_r(q) = q.k_hat_r/sqrt d + b_hat_r taken at
// reference queries q_hat_r: k_hat_r = Attn(q_hat_r, K_C, K_C) and
// b_hat_r = F(q_hat_r) - q_hat_r.k_hat_r/sqrt d.  Upper-level nodes merge their
// children's summaries the same way; with RoPE the parent's rotated reference
// query rescores the children, which adds 1/sqrt d <k_hat_{r,c}, q_hat_P - q_hat_c>
// to each child's own tangent value.  That sum is the child plane evaluated at
// q_hat_P, s_c = scale q_hat_P.k_hat_{r,c} + b_hat_{r,c}, which is what the
// parent kernel computes.  A level-1 node is added every C decode steps and a
// level-2 node every C^2 steps (append cadence, same section).
//
// Reference queries are rotated (rotate-half pairs (i, i+d/2), angle
// pos * base^(-2i/d), fp64 angles) to the node's first key position n * C^level.
// build_leaves_mfma takes the fp64 cosine and sine of each pair's angle,
// advanced from leaf to leaf by one fixed fp64 rotation, and applies the
// rotation in fp32; the other kernels compute the sine and cosine per node and
// rotate in fp64.
//
// Four kernels: build_leaves_mfma (bf16 keys, C in {16, 32, 64}): one wave per
// leaf on the matrix cores; build_leaves_small (bf16 keys, C in {2, 4, 8}): one
// wave per leaf, lanes over dimensions; build_leaves (other geometries): one
// workgroup per leaf, keys staged in LDS as fp32; build_parents: one wave per
// (node, plane) pair, the children's planes in registers.  b_hat is formed as
// F - sum_j w_j z_j, which equals F - scale q_hat.k_hat since k_hat = sum_j w_j k_j.
#include "zha_internal.hpp"

namespace zha {

struct BuildParams {
  const void* K;              // [BH][T_cap][d]
  const int64_t* T;           // [B]
  const float* qref;          // [H_kv][R][d]
  float* khat;                // level l:   [BH][ncap][R][d]
  float* bhat;                //            [BH][ncap][R]
  const float* khat_ch;       // level l-1: [BH][ncap_ch][R][d]
  const float* bhat_ch;
  int64_t ncap, ncap_ch;
  int64_t* n_built;           // [L][B]
  int32_t B, H_kv, d, C, R, level, rope, kv_dtype, append;
  float scale, rope_base;
  int64_t T_cap, span;        // span = C^level
};

// The R reference queries of a node whose first key is at position pos, rotated
// when P.rope, into qh[r][d] (row stride ld).
__device__ inline void load_ref_queries(const BuildParams& P, int h, int64_t pos,
                                        float* qh, int ld) {
  const int d = P.d, half = d / 2, R = P.R;
  const float* qr = P.qref + (int64_t)h * R * d;
  if (!P.rope) {
    for (int idx = threadIdx.x; idx < R * d; idx += blockDim.x)
      qh[(idx / d) * ld + idx % d] = qr[idx];
    return;
  }
  for (int idx = threadIdx.x; idx < R * half; idx += blockDim.x) {
    const int r = idx / half, i = idx % half;
    const double theta = pow((double)P.rope_base, -2.0 * (double)i / (double)d);
    const double ang = (double)pos * theta;
    double sn, cs;
    sincos(ang, &sn, &cs);
    const double x1 = qr[r * d + i], x2 = qr[r * d + i + half];
    qh[r * ld + i] = (float)(x1 * cs - x2 * sn);
    qh[r * ld + i + half] = (float)(x1 * sn + x2 * cs);
  }
}

constexpr int kMaxD = 128, kMaxC = 64, kMaxR = 16;

// LDS of build_leaves (one workgroup per leaf).
struct BuildSmem {
  float k[kMaxC][kMaxD + 1];     // the leaf's keys (fp32)
  float qh[kMaxR][kMaxD + 1];    // reference queries of the node
  float z[kMaxR][kMaxC];         // logits
  float w[kMaxR][kMaxC];         // softmax weights
  float F[kMaxR], wz[kMaxR];     // log-mass and sum_j w_j z_j
};

__device__ inline void node_range(const BuildParams& P, int b, int64_t& n0, int64_t& n1) {
  int64_t T = P.T[b];
  if (T < 0) T = 0;
  if (T > P.T_cap) T = P.T_cap;
  n1 = T / P.span;
  if (n1 > P.ncap) n1 = P.ncap;
  n0 = P.append ? P.n_built[(int64_t)(P.level - 1) * P.B + b] : 0;
  if (n0 < 0) n0 = 0;
  if (n0 > n1) n0 = n1;
}

// Softmax over the C logits of each plane: wave w handles planes w, w+4, ...
__device__ inline void plane_softmax(BuildSmem& sm, int R, int C) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int r = wave; r < R; r += (int)(blockDim.x >> 6)) {
    const float z = lane < C ? sm.z[r][lane] : -INFINITY;
    const float m = wave_max(z);
    const float e = lane < C ? expf(z - m) : 0.0f;
    const float s = wave_sum(e);
    const float w = e / s;
    const float wz = wave_sum(lane < C ? w * z : 0.0f);
    if (lane < C) sm.w[r][lane] = w;
    if (lane == 0) { sm.F[r] = m + logf(s); sm.wz[r] = wz; }
  }
}

__global__ void __launch_bounds__(256) build_leaves(BuildParams P) {
  __shared__ BuildSmem sm;
  const int gi = blockIdx.y;
  const int b = gi / P.H_kv, h = gi % P.H_kv;
  int64_t n0, n1;
  node_range(P, b, n0, n1);
  const int d = P.d, C = P.C, R = P.R;
  for (int64_t n = n0 + blockIdx.x; n < n1; n += gridDim.x) {
    // keys of the leaf -> LDS fp32
    const int64_t row0 = (int64_t)gi * P.T_cap + n * C;
    if (P.kv_dtype == ZHA_BF16) {
      const uint16_t* Kb = (const uint16_t*)P.K + row0 * d;
      for (int idx = threadIdx.x; idx < C * d / 2; idx += blockDim.x) {
        const uint32_t pr = ((const uint32_t*)Kb)[idx];
        const int e = idx * 2;
        sm.k[e / d][e % d] = bf16_lo(pr);
        sm.k[e / d][e % d + 1] = bf16_hi(pr);
      }
    } else {
      const float* Kf = (const float*)P.K + row0 * d;
      for (int idx = threadIdx.x; idx < C * d; idx += blockDim.x)
        sm.k[idx / d][idx % d] = Kf[idx];
    }
    load_ref_queries(P, h, n * C, &sm.qh[0][0], kMaxD + 1);
    __syncthreads();
    // logits z[r][j] = scale * q_hat_r . k_j; thread: key j = t % 64, planes t/64 + 4i
    {
      const int j = threadIdx.x & 63;
      const int r0 = threadIdx.x >> 6;
      if (j < C) {
        for (int r = r0; r < R; r += 4) {
          float acc = 0.0f;
          for (int c = 0; c < d; ++c) acc += sm.qh[r][c] * sm.k[j][c];
          sm.z[r][j] = acc * P.scale;
        }
      }
    }
    __syncthreads();
    plane_softmax(sm, R, C);
    __syncthreads();
    // k_hat[r][c] = sum_j w[r][j] k[j][c]
    float* kh = P.khat + (((int64_t)gi * P.ncap + n) * R) * d;
    for (int idx = threadIdx.x; idx < R * d; idx += blockDim.x) {
      const int r = idx / d, c = idx % d;
      float acc = 0.0f;
      for (int j = 0; j < C; ++j) acc += sm.w[r][j] * sm.k[j][c];
      kh[idx] = acc;
    }
    if (threadIdx.x < R)
      P.bhat[((int64_t)gi * P.ncap + n) * R + threadIdx.x] = sm.F[threadIdx.x] - sm.wz[threadIdx.x];
    __syncthreads();
  }
}

// ---------------------------------------------------------------- leaves on MFMA
//
// bf16 keys, C in {16, 32, 64}, R <= 16: both products of a leaf are dense
// contractions, Z = Q_hat K^T (R x C over d) and k_hat = softmax(Z) K (R x d over
// C), and run on MFMA 16x16x32 bf16.  The fp32 operand of each (the scaled
// reference queries, then the softmax weights) is split into three bf16 terms
// hi + mid + lo, which carry it to ~2^-24; the keys are exact in bf16; products
// accumulate in fp32.  Rows are the planes (padded to 16).  Z: wave w takes keys
// 16w..16w+15, its key operand read straight from the cache rows.  k_hat: wave w
// takes the 16-dim tiles w, w+4, ..., its key operand read from K^T staged in
// LDS.  Under RoPE the reference queries are rotated per leaf; the fp64 angle of
// each dimension pair, shared by the R planes, advances by one fixed rotation
// from leaf to leaf (a sincos only at a wave's first leaf).

typedef __bf16 bf16x8b_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4b_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4b_t __attribute__((__vector_size__(4 * sizeof(uint32_t))));

__device__ inline void split3(float x, __bf16& hi, __bf16& mid, __bf16& lo) {
  const uint16_t h = f32_to_bf16_rne(x);
  const float r1 = x - __uint_as_float((uint32_t)h << 16);
  const uint16_t m = f32_to_bf16_rne(r1);
  const float r2 = r1 - __uint_as_float((uint32_t)m << 16);
  const uint16_t l = f32_to_bf16_rne(r2);
  hi = __builtin_bit_cast(__bf16, h);
  mid = __builtin_bit_cast(__bf16, m);
  lo = __builtin_bit_cast(__bf16, l);
}

// Leaf summaries on the matrix cores, one wave per leaf (bf16 keys).
//   Z = Q_hat K^T          A = scaled reference queries (3-way bf16 split),
//                          B = the leaf's keys as loaded (row = key, 8 dims)
//   softmax over keys per plane in registers, b_hat = F - sum_j w_j z_j
//   k_hat^T = K^T W^T      A = K^T through LDS, B = W (3-way bf16 split)
// A wave loops over leaves with the next leaf's keys in flight; no workgroup
// barriers are needed (a workgroup is one wave).
template <int D, int C>
__global__ void __launch_bounds__(64) build_leaves_mfma(BuildParams P) {
  constexpr int KST = D / 32;              // dimension steps of Z
  constexpr int NT = C / 16;               // key tiles of Z
  constexpr int CK = C < 32 ? 32 : C;      // keys padded to whole contraction steps
  constexpr int KS2 = CK / 32;             // key steps of k_hat
  constexpr int KP = CK + 8;               // K^T row stride (bf16 elements)
  constexpr int WP = CK + 4;               // W row stride (floats)
  constexpr int H2 = D / 2;
  constexpr int KT_BYTES = D * KP * 2;
  static_assert(16 * (D + 4) * 4 <= KT_BYTES, "query staging aliases K^T");
  __shared__ __attribute__((aligned(16))) unsigned char lds[KT_BYTES + 16 * WP * 4];
  uint16_t (*kt)[KP] = reinterpret_cast<uint16_t (*)[KP]>(lds);
  float (*qs)[D + 4] = reinterpret_cast<float (*)[D + 4]>(lds);   // before K^T is written
  float (*wsm)[WP] = reinterpret_cast<float (*)[WP]>(lds + KT_BYTES);
  const int gi = blockIdx.y;
  const int b = gi / P.H_kv, h = gi % P.H_kv;
  const int lane = threadIdx.x, row = lane & 15, kg = lane >> 4;
  const int R = P.R;
  int64_t n0, n1;
  node_range(P, b, n0, n1);
  const float* qr = P.qref + (int64_t)h * R * D;
  // weights of the padded keys C..CK-1 stay zero
  for (int i = lane; i < 16 * WP; i += 64) (&wsm[0][0])[i] = 0.0f;
  // RoPE: lane handles frequency lane % (d/2) for every plane it stages
  double theta = 0.0;
  if (P.rope) theta = pow((double)P.rope_base, -2.0 * (double)(lane % H2) / (double)D);

  bf16x8b_t qa[3][KST];
  // (cs, sn): cos and sin of this lane's RoPE angle at the current leaf
  auto build_qa = [&](double cs, double sn) {
    __syncthreads();                       // the previous leaf's K^T reads are done
    if (!P.rope) {
      for (int i = lane; i < 16 * D; i += 64) {
        const int r = i / D, c = i % D;
        qs[r][c] = (r < R) ? qr[r * D + c] * P.scale : 0.0f;
      }
    } else {
      // the angle is fp64; the rotations run in fp32 (within an ulp or two of the
      // fp64-rounded result, far inside the builder's accuracy)
      const float cf = (float)cs, sf = (float)sn;
      for (int idx = lane; idx < 16 * H2; idx += 64) {
        const int r = idx / H2, c = idx % H2;   // c == lane % H2
        float x1 = 0.0f, x2 = 0.0f;
        if (r < R) {
          const float a = qr[r * D + c], bb = qr[r * D + c + H2];
          x1 = fmaf(a, cf, -bb * sf);
          x2 = fmaf(a, sf, bb * cf);
        }
        qs[r][c] = x1 * P.scale;
        qs[r][c + H2] = x2 * P.scale;
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KST; ++s) {
      bf16x8b_t a0, a1, a2;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        __bf16 x0, x1, x2;
        split3(qs[row][s * 32 + kg * 8 + j], x0, x1, x2);
        a0[j] = x0; a1[j] = x1; a2[j] = x2;
      }
      qa[0][s] = a0; qa[1][s] = a1; qa[2][s] = a2;
    }
    __syncthreads();                       // K^T may overwrite the staging now
  };
  if (!P.rope) build_qa(1.0, 0.0);

  // lane's share of a leaf: keys 16t + row, dimensions 32s + 8kg .. +8
  const uint16_t* Kb = (const uint16_t*)P.K;
  auto fetch = [&](int64_t n, u32x4b_t (&v)[NT][KST]) {
    const uint16_t* kr = Kb + ((int64_t)gi * P.T_cap + n * C + row) * D + kg * 8;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int s = 0; s < KST; ++s)
        v[t][s] = __builtin_nontemporal_load((const u32x4b_t*)(kr + t * 16 * D + s * 32));
  };
  u32x4b_t kv[NT][KST];
  // leaves n and n+1 share a line of b-hat: their workgroups share an XCD
  int64_t n = n0 + xcd_grouped_x();
  if (n < n1) fetch(n, kv);
  // RoPE angle of this lane's frequency at leaf n, advanced by the fixed step of
  // gridDim.x leaves per iteration with one fp64 rotation (the angle pos * theta,
  // pos = n C, to ~1e-14 over a few hundred steps) instead of a sincos per leaf
  double rc = 1.0, rs = 0.0, dc = 1.0, ds = 0.0;
  if (P.rope) {
    sincos((double)(n * C) * theta, &rs, &rc);
    sincos((double)((int64_t)gridDim.x * C) * theta, &ds, &dc);
  }
  for (; n < n1; n += gridDim.x) {
    if (P.rope) {
      build_qa(rc, rs);
      const double c2 = rc * dc - rs * ds, s2 = rs * dc + rc * ds;
      rc = c2;
      rs = s2;
    }
    // ---- Z: z[t][i] = logit of plane 4kg + i, key 16t + row
    f32x4b_t z[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      z[t] = f32x4b_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KST; ++s) {
        const bf16x8b_t kb = __builtin_bit_cast(bf16x8b_t, kv[t][s]);
        z[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[0][s], kb, z[t], 0, 0, 0);
        z[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[1][s], kb, z[t], 0, 0, 0);
        z[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[2][s], kb, z[t], 0, 0, 0);
      }
    }
    // ---- K^T into LDS (padded keys zero), then the next leaf's keys in flight
#pragma unroll
    for (int t = 0; t < CK / 16; ++t)
#pragma unroll
      for (int s = 0; s < KST; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x = t < NT ? kv[t < NT ? t : 0][s][e] : 0u;
          kt[32 * s + 8 * kg + 2 * e][16 * t + row] = (uint16_t)(x & 0xffffu);
          kt[32 * s + 8 * kg + 2 * e + 1][16 * t + row] = (uint16_t)(x >> 16);
        }
    if (n + gridDim.x < n1) fetch(n + gridDim.x, kv);
    // ---- softmax over the leaf's keys, per plane (16 lanes share a plane)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pl = 4 * kg + i;
      float M = z[0][i];
#pragma unroll
      for (int t = 1; t < NT; ++t) M = fmaxf(M, z[t][i]);
      M = fmaxf(M, __shfl_xor(M, 1, 64));
      M = fmaxf(M, __shfl_xor(M, 2, 64));
      M = fmaxf(M, __shfl_xor(M, 4, 64));
      M = fmaxf(M, __shfl_xor(M, 8, 64));
      float e[NT], S = 0.0f, SZ = 0.0f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        e[t] = expf(z[t][i] - M);
        S += e[t];
        SZ += e[t] * z[t][i];
      }
      S += __shfl_xor(S, 1, 64); SZ += __shfl_xor(SZ, 1, 64);
      S += __shfl_xor(S, 2, 64); SZ += __shfl_xor(SZ, 2, 64);
      S += __shfl_xor(S, 4, 64); SZ += __shfl_xor(SZ, 4, 64);
      S += __shfl_xor(S, 8, 64); SZ += __shfl_xor(SZ, 8, 64);
      // b_hat = F - sum_j w_j z_j, F = M + log S
      if (row == 0 && pl < R) P.bhat[((int64_t)gi * P.ncap + n) * R + pl] = (M + logf(S)) - SZ / S;
#pragma unroll
      for (int t = 0; t < NT; ++t) wsm[pl][16 * t + row] = e[t] / S;
    }
    __syncthreads();
    // ---- k_hat^T = K^T W^T; acc[i] = k_hat of plane row, dimension 16td + 4kg + i
    bf16x8b_t wb[3][KS2];
#pragma unroll
    for (int s = 0; s < KS2; ++s) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        __bf16 x0, x1, x2;
        split3(wsm[row][32 * s + 8 * kg + j], x0, x1, x2);
        wb[0][s][j] = x0; wb[1][s][j] = x1; wb[2][s][j] = x2;
      }
    }
    float* kh = P.khat + ((int64_t)gi * P.ncap + n) * R * D;
#pragma unroll
    for (int td = 0; td < D / 16; ++td) {
      f32x4b_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS2; ++s) {
        const bf16x8b_t ka = __builtin_bit_cast(bf16x8b_t,
                                                *(const u32x4b_t*)&kt[16 * td + row][32 * s + 8 * kg]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, wb[0][s], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, wb[1][s], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, wb[2][s], acc, 0, 0, 0);
      }
      if (row < R) *(float4*)(kh + (int64_t)row * D + 16 * td + 4 * kg) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();                       // K^T and W are reused by the next leaf
  }
}

// ---------------------------------------------------------------- leaves, small C
//
// bf16 keys, C in {2, 4, 8}, R <= 16: a leaf is too small for the matrix cores.
// One wave per leaf; lane l holds dimensions DPL l .. DPL l + DPL - 1 of the 16
// scaled reference queries (registers) and of the leaf's keys.  The planes go in
// passes of PP = 32 / CP (CP = max(C, 4) keys, the padding masked): a pass's 32
// partial dot products are summed over the 64 lanes by a halving butterfly
// (five rounds, then one plain exchange), which leaves lanes 2e and 2e+1 with
// entry e = plane * CP + key of the pass; the softmax of a plane runs over the
// lanes holding its keys; the weights pass through the wave's LDS to every lane,
// which forms its dimensions of k_hat for every plane.  The scaled queries sit
// in the wave's LDS (the passes index them at run time).  Same formulas as the
// MFMA kernel (b_hat = F - sum_j w_j z_j); the queries are rotated in fp64 here
// (one leaf per wave leaves no per-leaf staging to save) and then scaled.

// Lane l's N values: the lanes with bit DELTA set keep the upper half, the others
// the lower half, each adding its partner's copy of the half it keeps.
template <int N, int DELTA>
__device__ inline void halve_round(float* a, int lane) {
  const bool upper = (lane & DELTA) != 0;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float keep = upper ? a[i + N / 2] : a[i];
    const float send = upper ? a[i] : a[i + N / 2];
    a[i] = keep + __shfl_xor(send, DELTA, 64);
  }
}

template <int D, int CP>
__global__ void __launch_bounds__(256) build_leaves_small(BuildParams P) {
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(CP == 4 || CP == 8, "padded keys");
  constexpr int DPL = D / 64;             // dimensions per lane
  constexpr int PP = 32 / CP;             // planes per pass
  constexpr int H2 = D / 2;
  __shared__ float wsh[4][16][CP];        // per wave: the leaf's softmax weights
  __shared__ __attribute__((aligned(16))) float qsh[4][16][D];   // per wave: scaled queries
  const int gi = blockIdx.y;
  const int b = gi / P.H_kv, h = gi % P.H_kv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int C = P.C, R = P.R;
  int64_t n0, n1;
  node_range(P, b, n0, n1);
  const float* qr = P.qref + (int64_t)h * R * D;
  const int d0 = DPL * lane;
  // the 16 scaled reference queries at this lane's dimensions, into the wave's LDS
  float (*qv)[D] = qsh[wave];
  auto set_q = [&](int64_t pos) {
    if (!P.rope) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int k = 0; k < DPL; ++k) qv[r][d0 + k] = (r < R) ? qr[r * D + d0 + k] * P.scale : 0.0f;
      wave_lds_sync();
      return;
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int c = d0 + k, i = c < H2 ? c : c - H2;   // rotate-half pair (i, i + d/2)
      const double theta = pow((double)P.rope_base, -2.0 * (double)i / (double)D);
      double sn, cs;
      sincos((double)pos * theta, &sn, &cs);
#pragma unroll 2
      for (int r = 0; r < 16; ++r) {
        float x = 0.0f;
        if (r < R) {
          const double a = qr[r * D + i], bb = qr[r * D + i + H2];
          x = c < H2 ? (float)(a * cs - bb * sn) : (float)(a * sn + bb * cs);
        }
        qv[r][d0 + k] = x * P.scale;
      }
    }
    wave_lds_sync();
  };
  if (!P.rope) set_q(0);
  const uint16_t* Kb = (const uint16_t*)P.K;
  const int64_t nw = (int64_t)gridDim.x * 4;
  // after a pass's butterfly: entry e = lane / 2, plane PP pass + e / CP, key e % CP
  const int e = lane >> 1, jl = e % CP, rl = e / CP;
  for (int64_t n = n0 + (int64_t)xcd_grouped_x() * 4 + wave; n < n1; n += nw) {
    if (P.rope) set_q(n * C);              // (after the previous leaf's closing sync)
    // this lane's dimensions of the leaf's keys (padding keys zero)
    float kv[CP][DPL];
    const uint16_t* kr = Kb + ((int64_t)gi * P.T_cap + n * C) * D + d0;
#pragma unroll
    for (int j = 0; j < CP; ++j) {
      if constexpr (DPL == 2) {
        const uint32_t pr = j < C ? *(const uint32_t*)(kr + (int64_t)j * D) : 0u;
        kv[j][0] = bf16_lo(pr);
        kv[j][1] = bf16_hi(pr);
      } else {
        kv[j][0] = j < C ? __uint_as_float((uint32_t)kr[(int64_t)j * D] << 16) : 0.0f;
      }
    }
#pragma unroll 1
    for (int pass = 0; pass < 16 / PP; ++pass) {
      float a[32];
#pragma unroll
      for (int r = 0; r < PP; ++r) {
        float q[DPL];
#pragma unroll
        for (int k = 0; k < DPL; ++k) q[k] = qv[PP * pass + r][d0 + k];
#pragma unroll
        for (int j = 0; j < CP; ++j) {
          float acc = 0.0f;
#pragma unroll
          for (int k = 0; k < DPL; ++k) acc = fmaf(q[k], kv[j][k], acc);
          a[r * CP + j] = acc;
        }
      }
      halve_round<32, 32>(a, lane);
      halve_round<16, 16>(a, lane);
      halve_round<8, 8>(a, lane);
      halve_round<4, 4>(a, lane);
      halve_round<2, 2>(a, lane);
      const float zs = a[0] + __shfl_xor(a[0], 1, 64);
      // softmax of plane PP pass + rl over the lanes holding its keys (lane bits 1 .. log2 CP)
      const float z = jl < C ? zs : -INFINITY;
      float M = z;
#pragma unroll
      for (int m = 2; m < 2 * CP; m <<= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
      const float ex = jl < C ? expf(z - M) : 0.0f;
      float S = ex, SZ = jl < C ? ex * z : 0.0f;
#pragma unroll
      for (int m = 2; m < 2 * CP; m <<= 1) {
        S += __shfl_xor(S, m, 64);
        SZ += __shfl_xor(SZ, m, 64);
      }
      const int r = PP * pass + rl;
      // b_hat = F - sum_j w_j z_j, F = M + log S
      if ((lane & (2 * CP - 1)) == 0 && r < R)
        P.bhat[((int64_t)gi * P.ncap + n) * R + r] = (M + logf(S)) - SZ / S;
      if ((lane & 1) == 0) wsh[wave][r][jl] = ex / S;
    }
    wave_lds_sync();
    // k_hat of every plane at this lane's dimensions
    float* kh = P.khat + ((int64_t)gi * P.ncap + n) * R * D + d0;
#pragma unroll 2
    for (int rr = 0; rr < 16; ++rr) {
      if (rr < R) {
        float acc[DPL];
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] = 0.0f;
#pragma unroll
        for (int j = 0; j < CP; ++j) {
          const float w = wsh[wave][rr][j];      // the same address in every lane
#pragma unroll
          for (int k = 0; k < DPL; ++k) acc[k] = fmaf(w, kv[j][k], acc[k]);
        }
        if constexpr (DPL == 2) *(float2*)(kh + (int64_t)rr * D) = make_float2(acc[0], acc[1]);
        else kh[(int64_t)rr * D] = acc[0];
      }
    }
    wave_lds_sync();                       // the weights are rewritten by the next leaf
  }
}

// Parent summaries, one wave per (node, plane) pair: the children's planes r
// (child 4t + lane/16, dimensions (lane%16)*d/16 ..) stay in registers, and an
// exact two-pass softmax over the children gives k_hat and b_hat.  No LDS, no
// workgroup barriers.
template <int D, int MT>
__global__ void __launch_bounds__(256) build_parents(BuildParams P) {
  static_assert(MT >= 1 && 4 * MT <= kMaxC, "child rounds");
  constexpr int DPL = D / 16;              // dimensions per lane
  constexpr int NV = DPL / 4;              // float4 per child per lane
  constexpr int H2 = D / 2;                // MT: child rounds, ceil(C / 4)
  const int gi = blockIdx.y;
  const int b = gi / P.H_kv, h = gi % P.H_kv;
  const int lane = threadIdx.x & 63, cg = lane >> 4, ds = (lane & 15) * DPL;
  const int C = P.C, R = P.R;
  int64_t n0, n1;
  node_range(P, b, n0, n1);
  const float* qr = P.qref + (int64_t)h * R * D;
  // RoPE: lane computes frequency lane % (d/2) and shares it by shuffles
  double theta = 0.0;
  if (P.rope) theta = pow((double)P.rope_base, -2.0 * (double)(lane % H2) / (double)D);
  const int64_t npairs = (n1 - n0) * R;
  // the 32 pairs of one line of b-hat run in 8 workgroups on one XCD
  for (int64_t pr = (int64_t)xcd_grouped_x() * 4 + (threadIdx.x >> 6); pr < npairs;
       pr += (int64_t)gridDim.x * 4) {
    const int64_t n = n0 + pr / R;
    const int r = (int)(pr % R);
    const int64_t ch0 = n * C;
    float4 v[MT][NV];
    const float* src = P.khat_ch + (((int64_t)gi * P.ncap_ch + ch0 + cg) * R + r) * D + ds;
    const int64_t cstep = (int64_t)4 * R * D;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int q = 0; q < NV; ++q)
        v[t][q] = 4 * t + cg < C ? *(const float4*)(src + t * cstep + 4 * q)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
    const float bl = lane < C ? P.bhat_ch[((int64_t)gi * P.ncap_ch + ch0 + lane) * R + r] : 0.0f;
    // plane r's reference query at the node's first key position
    float qv[DPL];
    if (!P.rope) {
#pragma unroll
      for (int k = 0; k < DPL; ++k) qv[k] = qr[r * D + ds + k];
    } else {
      double sn, cs;
      sincos((double)(n * P.span) * theta, &sn, &cs);
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int c = ds + k, i = c < H2 ? c : c - H2;
        const double ci = __shfl(cs, i, 64), si = __shfl(sn, i, 64);
        const double x1 = qr[r * D + i], x2 = qr[r * D + i + H2];
        qv[k] = c < H2 ? (float)(x1 * ci - x2 * si) : (float)(x1 * si + x2 * ci);
      }
    }
    // logits s_j = scale q.k_hat_{r,j} + b_hat_{r,j}
    float sl[MT], dot[MT];
    float M = -INFINITY;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      float acc = 0.0f;
#pragma unroll
      for (int q = 0; q < NV; ++q) {
        acc = fmaf(v[t][q].x, qv[4 * q], acc);
        acc = fmaf(v[t][q].y, qv[4 * q + 1], acc);
        acc = fmaf(v[t][q].z, qv[4 * q + 2], acc);
        acc = fmaf(v[t][q].w, qv[4 * q + 3], acc);
      }
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      acc += __shfl_xor(acc, 4, 64);
      acc += __shfl_xor(acc, 8, 64);
      const int j = 4 * t + cg;
      const float bj = __shfl(bl, j, 64);
      dot[t] = acc * P.scale;
      sl[t] = j < C ? dot[t] + bj : -INFINITY;
      M = fmaxf(M, sl[t]);
    }
    M = fmaxf(M, __shfl_xor(M, 16, 64));
    M = fmaxf(M, __shfl_xor(M, 32, 64));
    float S = 0.0f, SW = 0.0f, ka[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) ka[k] = 0.0f;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float e = 4 * t + cg < C ? expf(sl[t] - M) : 0.0f;
      S += e;
      SW += e * dot[t];
#pragma unroll
      for (int q = 0; q < NV; ++q) {
        ka[4 * q] = fmaf(e, v[t][q].x, ka[4 * q]);
        ka[4 * q + 1] = fmaf(e, v[t][q].y, ka[4 * q + 1]);
        ka[4 * q + 2] = fmaf(e, v[t][q].z, ka[4 * q + 2]);
        ka[4 * q + 3] = fmaf(e, v[t][q].w, ka[4 * q + 3]);
      }
    }
    S += __shfl_xor(S, 16, 64);
    SW += __shfl_xor(SW, 16, 64);
    S += __shfl_xor(S, 32, 64);
    SW += __shfl_xor(SW, 32, 64);
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      ka[k] += __shfl_xor(ka[k], 16, 64);
      ka[k] += __shfl_xor(ka[k], 32, 64);
    }
    if (cg == 0) {
      float* kh = P.khat + (((int64_t)gi * P.ncap + n) * R + r) * D + ds;
#pragma unroll
      for (int q = 0; q < NV; ++q)
        *(float4*)(kh + 4 * q) = make_float4(ka[4 * q] / S, ka[4 * q + 1] / S,
                                             ka[4 * q + 2] / S, ka[4 * q + 3] / S);
    }
    // b_hat = F - sum_j w_j z_j with F = M + log S and z_j = scale q.k_hat_{r,j}
    if (lane == 0) P.bhat[((int64_t)gi * P.ncap + n) * R + r] = (M + logf(S)) - SW / S;
  }
}

// Record the built node counts once every build launch of the call is done.
__global__ void commit_levels(const int64_t* T, int64_t* n_built, int B, int C, int l0,
                              int l1, int64_t T_cap) {
  const int b = threadIdx.x + blockIdx.x * blockDim.x;
  if (b >= B) return;
  int64_t t = T[b];
  if (t < 0) t = 0;
  if (t > T_cap) t = T_cap;
  int64_t span = 1;
  for (int l = 1; l <= l1; ++l) {
    span *= C;
    if (l >= l0) n_built[(int64_t)(l - 1) * B + b] = t / span;
  }
}

static int32_t check_build(const zha_cfg* cfg, const zha_kv* kv, const float* qref,
                           const zha_tree* tree) {
  int32_t rc = zha_check_cfg(cfg);
  if (rc != ZHA_OK) return rc;
  if (kv == nullptr || kv->K == nullptr || kv->T == nullptr || qref == nullptr ||
      tree == nullptr || tree->n_built == nullptr)
    return ZHA_EINVAL;
  int64_t span = 1;
  for (int l = 1; l <= cfg->L; ++l) {
    span *= cfg->C;
    if (tree->khat[l - 1] == nullptr || tree->bhat[l - 1] == nullptr) return ZHA_EINVAL;
    if (tree->n_cap[l - 1] < cfg->T_cap / span) return ZHA_EINVAL;
  }
  return ZHA_OK;
}

static BuildParams make_params(const zha_cfg* cfg, const zha_kv* kv, const float* qref,
                               const zha_tree* tree, int level, int append) {
  BuildParams P;
  P.K = kv->K; P.T = kv->T; P.qref = qref;
  P.khat = tree->khat[level - 1]; P.bhat = tree->bhat[level - 1];
  P.ncap = tree->n_cap[level - 1];
  P.khat_ch = level > 1 ? tree->khat[level - 2] : nullptr;
  P.bhat_ch = level > 1 ? tree->bhat[level - 2] : nullptr;
  P.ncap_ch = level > 1 ? tree->n_cap[level - 2] : 0;
  P.n_built = tree->n_built;
  P.B = cfg->B; P.H_kv = cfg->H_kv; P.d = cfg->d; P.C = cfg->C; P.R = cfg->R;
  P.level = level; P.rope = cfg->rope; P.kv_dtype = cfg->kv_dtype; P.append = append;
  P.scale = cfg->scale; P.rope_base = cfg->rope_base;
  P.T_cap = cfg->T_cap;
  int64_t span = 1;
  for (int l = 0; l < level; ++l) span *= cfg->C;
  P.span = span;
  return P;
}

static void launch_level(const BuildParams& P, int64_t max_nodes, hipStream_t s) {
  int64_t gx = max_nodes < 1 ? 1 : max_nodes;
  if (gx > 65535) gx = 65535;
  const dim3 grid((unsigned)gx, (unsigned)(P.B * P.H_kv));
  // the MFMA leaf builder is one wave per workgroup looping over leaves: about
  // seven waves per compute unit in all (its LDS share allows seven)
  int64_t lx = (7 * 256 + P.B * P.H_kv - 1) / (P.B * P.H_kv);
  lx = (lx + 7) / 8 * 8;   // whole rounds of the XCDs
  const dim3 lgrid((unsigned)(gx < lx ? gx : lx), (unsigned)(P.B * P.H_kv));
  const bool mfma = P.kv_dtype == ZHA_BF16 && P.R <= 16 && (P.C == 16 || P.C == 32 || P.C == 64);
  const bool small = P.kv_dtype == ZHA_BF16 && P.R <= 16 && (P.C == 2 || P.C == 4 || P.C == 8);
  // small-C leaves: one wave per leaf, four per workgroup, about eight
  // workgroups per compute unit in all
  int64_t sx = (2048 + P.B * P.H_kv - 1) / (P.B * P.H_kv);
  sx = (sx + 7) / 8 * 8;
  const int64_t sw = (gx + 3) / 4;
  const dim3 sgrid((unsigned)(sw < sx ? sw : sx), (unsigned)(P.B * P.H_kv));
  // parents: one wave per (node, plane) pair, four waves per workgroup, about
  // four workgroups per compute unit in all
  const int64_t pw = (gx * P.R + 3) / 4;
  const int64_t pmax = ((1024 + P.B * P.H_kv - 1) / (P.B * P.H_kv) + 7) / 8 * 8;
  const dim3 pgrid((unsigned)(pw < pmax ? pw : pmax), (unsigned)(P.B * P.H_kv));
  if (P.level == 1 && mfma) {
    const auto k = P.d == 128 ? (P.C == 64 ? build_leaves_mfma<128, 64>
                                 : P.C == 32 ? build_leaves_mfma<128, 32> : build_leaves_mfma<128, 16>)
                              : (P.C == 64 ? build_leaves_mfma<64, 64>
                                 : P.C == 32 ? build_leaves_mfma<64, 32> : build_leaves_mfma<64, 16>);
    hipLaunchKernelGGL(k, lgrid, dim3(64), 0, s, P);
  } else if (P.level == 1 && small) {
    const auto k = P.d == 128 ? (P.C == 8 ? build_leaves_small<128, 8> : build_leaves_small<128, 4>)
                              : (P.C == 8 ? build_leaves_small<64, 8> : build_leaves_small<64, 4>);
    hipLaunchKernelGGL(k, sgrid, dim3(256), 0, s, P);
  } else if (P.level == 1) {
    hipLaunchKernelGGL(build_leaves, grid, dim3(256), 0, s, P);
  } else {
    // child rounds ceil(C / 4): the parents' registers and work follow C
    const int mt = (P.C + 3) / 4;
    const auto k = P.d == 128
        ? (mt <= 1 ? build_parents<128, 1> : mt <= 2 ? build_parents<128, 2> : mt <= 4 ? build_parents<128, 4>
           : mt <= 8 ? build_parents<128, 8> : build_parents<128, 16>)
        : (mt <= 1 ? build_parents<64, 1> : mt <= 2 ? build_parents<64, 2> : mt <= 4 ? build_parents<64, 4>
           : mt <= 8 ? build_parents<64, 8> : build_parents<64, 16>);
    hipLaunchKernelGGL(k, pgrid, dim3(256), 0, s, P);
  }
}

}  // namespace zha

extern "C" int32_t zha_build_level(const zha_cfg* cfg, int32_t level, const zha_kv* kv,
                                   const float* qref, const zha_tree* tree, void* ws,
                                   size_t ws_bytes, void* stream) {
  int32_t rc = zha::check_build(cfg, kv, qref, tree);
  if (rc != ZHA_OK) return rc;
  if (level < 1 || level > cfg->L) return ZHA_EINVAL;
  (void)ws; (void)ws_bytes;
  hipStream_t s = (hipStream_t)stream;
  zha::BuildParams P = zha::make_params(cfg, kv, qref, tree, level, 0);
  zha::launch_level(P, P.ncap, s);
  hipLaunchKernelGGL(zha::commit_levels, dim3((cfg->B + 63) / 64), dim3(64), 0, s, kv->T,
                     tree->n_built, cfg->B, cfg->C, level, level, cfg->T_cap);
  return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_EHIP;
}

extern "C" int32_t zha_append(const zha_cfg* cfg, const zha_kv* kv, const float* qref,
                              const zha_tree* tree, int64_t max_new_tokens, void* ws,
                              size_t ws_bytes, void* stream) {
  int32_t rc = zha::check_build(cfg, kv, qref, tree);
  if (rc != ZHA_OK) return rc;
  if (max_new_tokens < 0) return ZHA_EINVAL;
  (void)ws; (void)ws_bytes;
  hipStream_t s = (hipStream_t)stream;
  int64_t span = 1;
  for (int level = 1; level <= cfg->L; ++level) {
    span *= cfg->C;
    zha::BuildParams P = zha::make_params(cfg, kv, qref, tree, level, 1);
    const int64_t bound = max_new_tokens / span + 1;
    zha::launch_level(P, bound < P.ncap ? bound : P.ncap, s);
  }
  hipLaunchKernelGGL(zha::commit_levels, dim3((cfg->B + 63) / 64), dim3(64), 0, s, kv->T,
                     tree->n_built, cfg->B, cfg->C, 1, cfg->L, cfg->T_cap);
  return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_EHIP;
}
