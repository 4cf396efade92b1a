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
//
// One workgroup builds one node (all R planes) at a time, staging the node's
// keys (or its children's compressed keys) in LDS as fp32.  b_hat is formed as
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

// Reference queries r0 .. r1-1 of node n at `level`, rotated when P.rope, into
// qh[r][d] (row stride ld).
__device__ inline void load_ref_queries(const BuildParams& P, int h, int64_t pos,
                                        float* qh, int ld, int r0 = 0, int r1 = -1) {
  const int d = P.d, half = d / 2;
  if (r1 < 0) r1 = P.R;
  const int nr = r1 - r0;
  const float* qr = P.qref + (int64_t)h * P.R * d;
  if (!P.rope) {
    for (int idx = threadIdx.x; idx < nr * d; idx += blockDim.x)
      qh[(r0 + idx / d) * ld + idx % d] = qr[r0 * d + idx];
    return;
  }
  for (int idx = threadIdx.x; idx < nr * half; idx += blockDim.x) {
    const int r = r0 + idx / half, i = idx % half;
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

struct BuildSmem {
  float k[kMaxC][kMaxD + 1];     // node keys (leaf) or one plane of child keys
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
// LDS.  Under RoPE the reference queries are rotated per leaf, with one fp64
// sincos per dimension pair shared by the R planes.

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

template <int D, int C>
__global__ void __launch_bounds__(256) build_leaves_mfma(BuildParams P) {
  constexpr int KST = D / 32;              // contraction steps of Z
  constexpr int KP = kMaxC + 8;            // key stride of K^T in LDS (bf16 elements)
  constexpr int NTZ = C / 16;              // key tiles of Z, one per wave
  constexpr int KSTEPS = (C + 31) / 32;    // contraction steps of W K
  __shared__ __attribute__((aligned(16))) uint16_t kt[D][KP];   // K^T (bf16 bits)
  __shared__ __attribute__((aligned(16))) float wsm[16][kMaxC + 4];   // softmax weights
  __shared__ float qs[16][D + 4];          // scaled (rotated) reference queries
  __shared__ float rc[D / 2], rsn[D / 2];  // RoPE cos / sin of the leaf position
  __shared__ float red[3][4][16];          // per-wave plane max, sum, sum w z
  const int gi = blockIdx.y;
  const int b = gi / P.H_kv, h = gi % P.H_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = P.R;
  int64_t n0, n1;
  node_range(P, b, n0, n1);
  const float* qr = P.qref + (int64_t)h * R * D;

  // keys C..31 of K^T stay zero (the 32-key contraction step pads short leaves)
  for (int i = tid; i < D * KP; i += 256) (&kt[0][0])[i] = 0;
  if (C < 32)                              // and so do their weights
    for (int i = tid; i < 16 * (kMaxC + 4); i += 256) (&wsm[0][0])[i] = 0.0f;
  auto stage_queries = [&](int64_t pos) {
    if (!P.rope) {
      for (int i = tid; i < 16 * D; i += 256) {
        const int r = i / D, c = i % D;
        qs[r][c] = (r < R) ? qr[r * D + c] * P.scale : 0.0f;
      }
      return;
    }
    constexpr int H2 = D / 2;
    if (tid < H2) {
      const double theta = pow((double)P.rope_base, -2.0 * (double)tid / (double)D);
      double sn, cs;
      sincos((double)pos * theta, &sn, &cs);
      rc[tid] = (float)cs;
      rsn[tid] = (float)sn;
    }
    __syncthreads();
    for (int i = tid; i < 16 * H2; i += 256) {
      const int r = i / H2, c = i % H2;
      float x1 = 0.0f, x2 = 0.0f;
      if (r < R) {
        const double a = qr[r * D + c], bb = qr[r * D + c + H2];
        const double cs = rc[c], sn = rsn[c];
        x1 = (float)(a * cs - bb * sn);
        x2 = (float)(a * sn + bb * cs);
      }
      qs[r][c] = x1 * P.scale;
      qs[r][c + H2] = x2 * P.scale;
    }
  };
  bf16x8b_t qa[3][KST];
  auto load_qa = [&]() {
    const int row = lane & 15, kg = lane >> 4;
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
  };
  if (!P.rope) {
    stage_queries(0);
    __syncthreads();
    load_qa();
  }
  // Wave w < C/16 owns keys 16w + (lane % 16); its MFMA B operand of step s is
  // the 8 dimensions 32s + 8(lane / 16).. of that key.  The same registers fill
  // K^T in LDS.  Two register sets alternate between leaves, so the keys of the
  // next two leaves are in flight while one is summarised.
  const uint16_t* Kb = (const uint16_t*)P.K;
  const int krow = 16 * wave + (lane & 15), kg0 = lane >> 4;
  const int64_t g = gridDim.x;
  auto fetch = [&](int64_t n, u32x4b_t (&v)[KST]) {
    if (wave >= NTZ || n >= n1) return;
    const uint16_t* kr = Kb + ((int64_t)gi * P.T_cap + n * C + krow) * D + kg0 * 8;
#pragma unroll
    for (int s = 0; s < KST; ++s) v[s] = __builtin_nontemporal_load((const u32x4b_t*)(kr + s * 32));
  };
  auto leaf = [&](int64_t n, u32x4b_t (&kv)[KST]) {
    __syncthreads();                       // the previous leaf's LDS reads are done
    if (P.rope) stage_queries(n * C);
    if (wave < NTZ) {
#pragma unroll
      for (int s = 0; s < KST; ++s) {
        const int c0 = 32 * s + 8 * kg0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kt[c0 + 2 * e][krow] = (uint16_t)(kv[s][e] & 0xffffu);
          kt[c0 + 2 * e + 1][krow] = (uint16_t)(kv[s][e] >> 16);
        }
      }
    }
    if (P.rope) {
      __syncthreads();
      load_qa();
    }
    // ---- Z = Q_hat K^T: z[i] is plane 4(lane/16)+i, key 16w + lane%16
    f32x4b_t z = {0.f, 0.f, 0.f, 0.f};
    if (wave < NTZ) {
#pragma unroll
      for (int s = 0; s < KST; ++s) {
        const bf16x8b_t kb = __builtin_bit_cast(bf16x8b_t, kv[s]);
        z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[0][s], kb, z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[1][s], kb, z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[2][s], kb, z, 0, 0, 0);
      }
    }
    fetch(n + 2 * g, kv);                  // this register set's next leaf
    if (wave < NTZ) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {        // per-wave max over its 16 keys
        float m = z[i];
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        m = fmaxf(m, __shfl_xor(m, 4, 64));
        m = fmaxf(m, __shfl_xor(m, 8, 64));
        if ((lane & 15) == 0) red[0][wave][4 * (lane >> 4) + i] = m;
      }
    }
    __syncthreads();
    float e4[4];
    if (wave < NTZ) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pl = 4 * (lane >> 4) + i;
        float M = red[0][0][pl];
#pragma unroll
        for (int w = 1; w < NTZ; ++w) M = fmaxf(M, red[0][w][pl]);
        const float e = expf(z[i] - M);
        e4[i] = e;
        float sm = e, sz = e * z[i];
        sm += __shfl_xor(sm, 1, 64); sz += __shfl_xor(sz, 1, 64);
        sm += __shfl_xor(sm, 2, 64); sz += __shfl_xor(sz, 2, 64);
        sm += __shfl_xor(sm, 4, 64); sz += __shfl_xor(sz, 4, 64);
        sm += __shfl_xor(sm, 8, 64); sz += __shfl_xor(sz, 8, 64);
        if ((lane & 15) == 0) { red[1][wave][pl] = sm; red[2][wave][pl] = sz; }
      }
    }
    __syncthreads();
    if (wave < NTZ) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pl = 4 * (lane >> 4) + i;
        float S = 0.0f;
#pragma unroll
        for (int w = 0; w < NTZ; ++w) S += red[1][w][pl];
        wsm[pl][16 * wave + (lane & 15)] = e4[i] / S;
      }
    }
    if (tid < R) {
      float M = red[0][0][tid], S = 0.0f, SZ = 0.0f;
#pragma unroll
      for (int w = 1; w < NTZ; ++w) M = fmaxf(M, red[0][w][tid]);
#pragma unroll
      for (int w = 0; w < NTZ; ++w) { S += red[1][w][tid]; SZ += red[2][w][tid]; }
      // b_hat = F - sum_j w_j z_j, F = M + log S
      P.bhat[((int64_t)gi * P.ncap + n) * R + tid] = (M + logf(S)) - SZ / S;
    }
    __syncthreads();
    // ---- k_hat = W K: wave w, 16-dim tiles w, w + 4, ...
    const int row = lane & 15, kg = lane >> 4;
    float* kh = P.khat + ((int64_t)gi * P.ncap + n) * R * D;
#pragma unroll
    for (int t = wave; t < D / 16; t += 4) {
      f32x4b_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        bf16x8b_t a0, a1, a2;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          __bf16 x0, x1, x2;
          split3(wsm[row][s * 32 + kg * 8 + j], x0, x1, x2);
          a0[j] = x0; a1[j] = x1; a2[j] = x2;
        }
        const bf16x8b_t kb = __builtin_bit_cast(bf16x8b_t,
                                                *(const u32x4b_t*)&kt[t * 16 + row][s * 32 + kg * 8]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, kb, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, kb, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, kb, acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pl = 4 * kg + i;
        if (pl < R) kh[(int64_t)pl * D + t * 16 + row] = acc[i];
      }
    }
  };
  u32x4b_t ka[KST], kb2[KST];
  const int64_t first = n0 + blockIdx.x;
  fetch(first, ka);
  fetch(first + g, kb2);
  for (int64_t n = first; n < n1; n += 2 * g) {
    leaf(n, ka);
    if (n + g < n1) leaf(n + g, kb2);
  }
}

__global__ void __launch_bounds__(256) build_parents(BuildParams P) {
  __shared__ BuildSmem sm;
  const int gi = blockIdx.y;
  const int b = gi / P.H_kv, h = gi % P.H_kv;
  int64_t n0, n1;
  node_range(P, b, n0, n1);
  const int d = P.d, C = P.C, R = P.R;
  // one (node, plane) pair at a time: planes of a node are independent
  for (int64_t pr = blockIdx.x; pr < (n1 - n0) * R; pr += gridDim.x) {
    const int64_t n = n0 + pr / R;
    const int r = (int)(pr % R);
    __syncthreads();                      // the previous pair's LDS reads are done
    load_ref_queries(P, h, n * P.span, &sm.qh[0][0], kMaxD + 1, r, r + 1);
    const int64_t ch0 = n * C;   // first child
    {
      // children's plane r -> LDS: 16-byte loads (d is 64 or 128), all of a
      // thread's loads (at most 8) in flight before its stores
      {
        // 256 is a multiple of d/4, so a thread keeps its column and steps rows
        constexpr int IT = kMaxC * kMaxD / 4 / 256;
        const int dq = d / 4, rstep = 256 / dq;
        const int j0 = threadIdx.x / dq, c = 4 * (threadIdx.x % dq);
        const float* src = P.khat_ch + (((int64_t)gi * P.ncap_ch + ch0 + j0) * R + r) * d + c;
        const int64_t step = (int64_t)rstep * R * d;
        float4 v[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it)
          if (j0 + it * rstep < C) v[it] = *(const float4*)(src + it * step);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          const int j = j0 + it * rstep;
          if (j < C) {
            sm.k[j][c] = v[it].x;
            sm.k[j][c + 1] = v[it].y;
            sm.k[j][c + 2] = v[it].z;
            sm.k[j][c + 3] = v[it].w;
          }
        }
      }
      __syncthreads();
      // s_j = scale q_hat_P . k_hat_{r,j} + b_hat_{r,j}: 4 waves split d, then sum
      {
        const int j = threadIdx.x & 63, part = threadIdx.x >> 6;
        const int cq = d / 4;
        float acc = 0.0f;
        if (j < C)
          for (int c = part * cq; c < (part + 1) * cq; ++c) acc += sm.qh[r][c] * sm.k[j][c];
        sm.w[part][j] = acc;  // scratch (reused below)
      }
      __syncthreads();
      if (threadIdx.x < 64) {
        const int j = threadIdx.x;
        float s = -INFINITY, dot = 0.0f;
        if (j < C) {
          dot = (sm.w[0][j] + sm.w[1][j]) + (sm.w[2][j] + sm.w[3][j]);
          s = dot * P.scale + P.bhat_ch[((int64_t)gi * P.ncap_ch + ch0 + j) * R + r];
        }
        const float m = wave_max(s);
        const float e = j < C ? expf(s - m) : 0.0f;
        const float sum = wave_sum(e);
        const float w = e / sum;
        const float wdot = wave_sum(j < C ? w * dot * P.scale : 0.0f);
        if (j < C) sm.z[0][j] = w;
        if (j == 0) { sm.F[0] = m + logf(sum); sm.wz[0] = wdot; }
      }
      __syncthreads();
      float* kh = P.khat + (((int64_t)gi * P.ncap + n) * R + r) * d;
      for (int c = threadIdx.x; c < d; c += blockDim.x) {
        float acc = 0.0f;
        for (int j = 0; j < C; ++j) acc += sm.z[0][j] * sm.k[j][c];
        kh[c] = acc;
      }
      if (threadIdx.x == 0)
        P.bhat[((int64_t)gi * P.ncap + n) * R + r] = sm.F[0] - sm.wz[0];
      __syncthreads();
    }
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
  // the MFMA leaf builder loops over leaves with a prefetch: about two
  // workgroups per compute unit in all (its register budget allows two)
  const int64_t lx = (512 + P.B * P.H_kv - 1) / (P.B * P.H_kv);
  const dim3 lgrid((unsigned)(gx < lx ? gx : lx), (unsigned)(P.B * P.H_kv));
  const bool mfma = P.kv_dtype == ZHA_BF16 && P.R <= 16 && (P.C == 16 || P.C == 32 || P.C == 64);
  // parents are built one (node, plane) pair per workgroup iteration
  const dim3 pgrid((unsigned)(gx * P.R > 65535 ? 65535 : gx * P.R), (unsigned)(P.B * P.H_kv));
  if (P.level == 1 && mfma) {
    const auto k = P.d == 128 ? (P.C == 64 ? build_leaves_mfma<128, 64>
                                 : P.C == 32 ? build_leaves_mfma<128, 32> : build_leaves_mfma<128, 16>)
                              : (P.C == 64 ? build_leaves_mfma<64, 64>
                                 : P.C == 32 ? build_leaves_mfma<64, 32> : build_leaves_mfma<64, 16>);
    hipLaunchKernelGGL(k, lgrid, dim3(256), 0, s, P);
  } else if (P.level == 1)
    hipLaunchKernelGGL(build_leaves, grid, dim3(256), 0, s, P);
  else
    hipLaunchKernelGGL(build_parents, pgrid, dim3(256), 0, s, P);
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
