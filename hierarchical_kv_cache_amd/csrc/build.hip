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
  uint16_t* khat16;           //            bf16 copy of khat, or null
  const float* khat_ch;       // level l-1: [BH][ncap_ch][R][d]
  const float* bhat_ch;
  int64_t ncap, ncap_ch;
  int64_t* n_built;           // [L][B]
  int32_t B, H_kv, d, C, R, level, rope, kv_dtype, append;
  float scale, rope_base;
  int64_t T_cap, span;        // span = C^level
};

// The bf16 copy of k_hat that routing may read (zha_tree.khat16): each value
// rounded to nearest even (the summaries are finite).
__device__ inline uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ inline void store_bf16x4(uint16_t* p, float a, float b, float c, float d) {
  uint2 v;
  v.x = bf16_bits(a) | (bf16_bits(b) << 16);
  v.y = bf16_bits(c) | (bf16_bits(d) << 16);
  *(uint2*)p = v;
}
__device__ inline void store_bf16x2(uint16_t* p, float a, float b) {
  *(uint32_t*)p = bf16_bits(a) | (bf16_bits(b) << 16);
}

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

// One leaf of sequence-head gi (head h) summarised by a whole workgroup of
// kGenericThreads threads: keys and reference queries staged in LDS as fp32.
constexpr int kGenericThreads = 256;

__device__ inline void generic_leaf(const BuildParams& P, BuildSmem& sm, int gi, int h, int64_t n) {
  constexpr int NW = kGenericThreads / kWave;
  const int d = P.d, C = P.C, R = P.R;
  // keys of the leaf -> LDS fp32
  const int64_t row0 = (int64_t)gi * P.T_cap + n * C;
  if (P.kv_dtype == ZHA_BF16) {
    const uint16_t* Kb = (const uint16_t*)P.K + row0 * d;
    for (int idx = threadIdx.x; idx < C * d / 2; idx += kGenericThreads) {
      const uint32_t pr = ((const uint32_t*)Kb)[idx];
      const int e = idx * 2;
      sm.k[e / d][e % d] = bf16_lo(pr);
      sm.k[e / d][e % d + 1] = bf16_hi(pr);
    }
  } else {
    const float* Kf = (const float*)P.K + row0 * d;
    for (int idx = threadIdx.x; idx < C * d; idx += kGenericThreads)
      sm.k[idx / d][idx % d] = Kf[idx];
  }
  load_ref_queries(P, h, n * C, &sm.qh[0][0], kMaxD + 1);
  __syncthreads();
  // logits z[r][j] = scale * q_hat_r . k_j; thread: key j = t % 64, planes t/64 + NW i
  {
    const int j = threadIdx.x & 63;
    const int r0 = threadIdx.x >> 6;
    if (j < C) {
      for (int r = r0; r < R; r += NW) {
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
  uint16_t* kh16 = P.khat16 ? P.khat16 + (((int64_t)gi * P.ncap + n) * R) * d : nullptr;
  for (int idx = threadIdx.x; idx < R * d; idx += kGenericThreads) {
    const int r = idx / d, c = idx % d;
    float acc = 0.0f;
    for (int j = 0; j < C; ++j) acc += sm.w[r][j] * sm.k[j][c];
    kh[idx] = acc;
    if (kh16) kh16[idx] = (uint16_t)bf16_bits(acc);
  }
  if (threadIdx.x < R)
    P.bhat[((int64_t)gi * P.ncap + n) * R + threadIdx.x] = sm.F[threadIdx.x] - sm.wz[threadIdx.x];
  __syncthreads();
}

__global__ void __launch_bounds__(kGenericThreads) build_leaves(BuildParams P) {
  __shared__ BuildSmem sm;
  const int gi = blockIdx.y;
  const int b = gi / P.H_kv, h = gi % P.H_kv;
  int64_t n0, n1;
  node_range(P, b, n0, n1);
  for (int64_t n = n0 + blockIdx.x; n < n1; n += gridDim.x) generic_leaf(P, sm, gi, h, n);
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
//   k_hat^T = K^T W^T      MFMA 16x16x16: A = 16 dims x 16 keys of K^T, read
//                          from the keys as stored in LDS (row = key) by the
//                          transposing LDS read; B = W^T (3-way bf16 split)
// The wave's LDS (kLds bytes) holds the keys and W; the query staging aliases
// the keys.  Only the wave's own lanes touch it, so wave-level LDS syncs order it.
template <int D, int C>
struct MfmaLeaf {
  static constexpr int KST = D / 32;              // dimension steps of Z
  static constexpr int NT = C / 16;               // key tiles of Z, key blocks of k_hat
  static constexpr int KRP = D + 16;              // key row stride in LDS (bf16 elements)
  static constexpr int WP = C + 4;                // W row stride (floats)
  static constexpr int H2 = D / 2;
  static constexpr int KR_BYTES = C * KRP * 2;
  static constexpr int QS_BYTES = 16 * (D + 4) * 4;
  static constexpr int KT_BYTES = KR_BYTES > QS_BYTES ? KR_BYTES : QS_BYTES;
  static constexpr int kLds = KT_BYTES + 16 * WP * 4;
  typedef u32x4b_t Keys[NT][KST];
  typedef bf16x8b_t QOps[3][KST];
  typedef short bf16x4s_t __attribute__((ext_vector_type(4)));   // bf16 bits

  __device__ static void init(unsigned char* lds, int lane) {
    float* wsm = reinterpret_cast<float*>(lds + KT_BYTES);
    for (int i = lane; i < 16 * WP; i += 64) wsm[i] = 0.0f;
  }

  // The scaled reference queries of head h as split MFMA A operands; under RoPE
  // rotated by the angle whose cosine and sine (of this lane's frequency,
  // lane % (d/2)) are cs and sn.
  __device__ static void build_qa(const BuildParams& P, int h, double cs, double sn,
                                  unsigned char* lds, QOps& qa, int lane) {
    float (*qs)[D + 4] = reinterpret_cast<float (*)[D + 4]>(lds);
    const int row = lane & 15, kg = lane >> 4;
    const int R = P.R;
    const float* qr = P.qref + (int64_t)h * R * D;
    wave_lds_sync();                       // the previous leaf's K^T reads are done
    if (!P.rope) {
      // float4 pieces, lane l taking pieces l + 64 i: every piece is loaded (a
      // padding row reads the last real row and is scaled by zero), so all the
      // loads are in flight at once instead of each waiting behind a branch on R
      constexpr int Q4 = 16 * D / 4, RQ = D / 4;
#pragma unroll
      for (int i = lane; i < Q4; i += 64) {
        const int r = i / RQ, c = (i % RQ) * 4;
        const bool real = r < R;
        const float f = real ? P.scale : 0.0f;   // padding rows are scaled to zero
        float4 x = *(const float4*)(qr + (real ? r : R - 1) * D + c);
        x.x *= f; x.y *= f; x.z *= f; x.w *= f;
        *(float4*)&qs[r][c] = x;
      }
    } else {
      // the angle is fp64; the rotations run in fp32 (within an ulp or two of the
      // fp64-rounded result, far inside the builder's accuracy)
      const float cf = (float)cs, sf = (float)sn;
      for (int idx = lane; idx < 16 * H2; idx += 64) {
        const int r = idx / H2, c = idx % H2;   // c == lane % H2
        const int rr = r < R ? r : R - 1;
        const float a = qr[rr * D + c], bb = qr[rr * D + c + H2];
        float x1 = 0.0f, x2 = 0.0f;
        if (r < R) {
          x1 = fmaf(a, cf, -bb * sf);
          x2 = fmaf(a, sf, bb * cf);
        }
        qs[r][c] = x1 * P.scale;
        qs[r][c + H2] = x2 * P.scale;
      }
    }
    wave_lds_sync();
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
    wave_lds_sync();                       // K^T may overwrite the staging now
  }

  // This lane's share of leaf n's keys: keys 16t + row, dimensions 32s + 8kg .. +8.
  __device__ static void fetch(const BuildParams& P, int gi, int64_t n, Keys& v, int lane) {
    const int row = lane & 15, kg = lane >> 4;
    const uint16_t* kr = (const uint16_t*)P.K + ((int64_t)gi * P.T_cap + n * C + row) * D + kg * 8;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int s = 0; s < KST; ++s)
        v[t][s] = __builtin_nontemporal_load((const u32x4b_t*)(kr + t * 16 * D + s * 32));
  }

  // Leaf n of sequence-head gi from its keys kv.  `next` is called once K^T is
  // in LDS and kv is free, to put the following leaf's keys in flight.
  template <class Next>
  __device__ static void leaf(const BuildParams& P, int gi, int64_t n, Keys& kv, const QOps& qa,
                              unsigned char* lds, int lane, Next&& next) {
    uint16_t (*kr)[KRP] = reinterpret_cast<uint16_t (*)[KRP]>(lds);
    float (*wsm)[WP] = reinterpret_cast<float (*)[WP]>(lds + KT_BYTES);
    const int row = lane & 15, kg = lane >> 4;
    const int R = P.R;
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
    // ---- the keys into LDS as loaded (a key's 8 dims per 16-byte store), then
    // the next leaf's keys in flight
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int s = 0; s < KST; ++s)
        *(u32x4b_t*)&kr[16 * t + row][32 * s + 8 * kg] = kv[t][s];
    next();
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
    wave_lds_sync();
    // ---- k_hat^T = K^T W^T; acc[i] = k_hat of plane row, dimension 16td + 4kg + i.
    // B: this lane's plane (row) at keys 16kb + 4kg .. +3, split three ways
    bf16x4s_t wb[3][NT];
#pragma unroll
    for (int kb = 0; kb < NT; ++kb) {
      const float4 w4 = *(const float4*)&wsm[row][16 * kb + 4 * kg];
      const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        __bf16 x0, x1, x2;
        split3(wv[j], x0, x1, x2);
        wb[0][kb][j] = __builtin_bit_cast(short, x0);
        wb[1][kb][j] = __builtin_bit_cast(short, x1);
        wb[2][kb][j] = __builtin_bit_cast(short, x2);
      }
    }
    typedef __attribute__((address_space(3))) __bf16 lds_bf16_t;
    typedef __bf16 bf16x4v_t __attribute__((__vector_size__(4 * sizeof(__bf16))));
    typedef __attribute__((address_space(3))) bf16x4v_t lds_bf16x4_t;
    float* kh = P.khat + ((int64_t)gi * P.ncap + n) * R * D;
#pragma unroll
    for (int td = 0; td < D / 16; ++td) {
      f32x4b_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NT; ++kb) {
        // A: dims 16td + row, keys 16kb + 4kg .. +3 of the stored keys, transposed
        lds_bf16x4_t* src = (lds_bf16x4_t*)(lds_bf16_t*)(&kr[16 * kb + (lane >> 2)][16 * td + 4 * (lane & 3)]);
        const bf16x4s_t ka = __builtin_bit_cast(bf16x4s_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(src));
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, wb[0][kb], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, wb[1][kb], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, wb[2][kb], acc, 0, 0, 0);
      }
      if (row < R) {
        *(float4*)(kh + (int64_t)row * D + 16 * td + 4 * kg) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        if (P.khat16)
          store_bf16x4(P.khat16 + ((int64_t)gi * P.ncap + n) * R * D + (int64_t)row * D + 16 * td + 4 * kg,
                       acc[0], acc[1], acc[2], acc[3]);
      }
    }
    wave_lds_sync();                       // K^T and W are reused by the next leaf
  }
};

// Prefill: one wave per workgroup loops over leaves with the next leaf's keys in
// flight.  Under RoPE the reference queries are rotated per leaf; the fp64 angle
// of each dimension pair, shared by the R planes, advances by one fixed rotation
// from leaf to leaf (a sincos only at a wave's first leaf).
template <int D, int C>
__global__ void __launch_bounds__(64) build_leaves_mfma(BuildParams P) {
  using M = MfmaLeaf<D, C>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[M::kLds];
  const int gi = blockIdx.y;
  const int b = gi / P.H_kv, h = gi % P.H_kv;
  const int lane = threadIdx.x;
  int64_t n0, n1;
  node_range(P, b, n0, n1);
  M::init(lds, lane);
  // RoPE: lane handles frequency lane % (d/2) for every plane it stages
  double theta = 0.0;
  if (P.rope) theta = pow((double)P.rope_base, -2.0 * (double)(lane % M::H2) / (double)D);
  typename M::QOps qa;
  if (!P.rope) M::build_qa(P, h, 1.0, 0.0, lds, qa, lane);
  typename M::Keys kv;
  // leaves n and n+1 share a line of b-hat: their workgroups share an XCD
  int64_t n = n0 + xcd_grouped_x();
  if (n < n1) M::fetch(P, gi, n, kv, lane);
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
      M::build_qa(P, h, rc, rs, lds, qa, lane);
      const double c2 = rc * dc - rs * ds, s2 = rs * dc + rc * ds;
      rc = c2;
      rs = s2;
    }
    const int64_t nn = n + gridDim.x;
    M::leaf(P, gi, n, kv, qa, lds, lane, [&] { if (nn < n1) M::fetch(P, gi, nn, kv, lane); });
  }
}

// ---------------------------------------------------------------- leaves, small C
//
// bf16 keys, C in {2, 4, 8}, R <= 16: a leaf is too small for the matrix cores.
// One wave per leaf; lane l holds dimensions DPL l .. DPL l + DPL - 1 of the
// leaf's keys (registers) and reads the same dimensions of the 16 scaled
// reference queries from the wave's LDS.  The planes go in passes of
// PP = 32 / CP (CP = max(C, 4) keys; a padding key repeats the last real one and
// gets weight zero): a pass's 32
// partial dot products are summed over the 64 lanes by a halving butterfly
// (five rounds, then one plain exchange), which leaves lanes 2e and 2e+1 with
// entry e = plane * CP + key of the pass; the softmax of a plane runs over the
// lanes holding its keys; the weights pass through the wave's LDS to every lane,
// which forms its dimensions of k_hat for every plane (the passes index the
// queries at run time, hence LDS rather than registers).  Same formulas as the
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

// Reference queries under RoPE for the small-C leaves, in two steps shared by
// the one-wave leaf and the plane-per-wave append, so the two round alike: the
// fp64 angle of dimension c at position pos (rotate-half pairs (i, i + d/2)),
// then dimension c of a row rotated by it and scaled.
template <int D>
__device__ inline void small_rope_angle(int c, int64_t pos, double rope_base, double& cs,
                                        double& sn) {
  const int i = c < D / 2 ? c : c - D / 2;
  const double theta = pow(rope_base, -2.0 * (double)i / (double)D);
  sincos((double)pos * theta, &sn, &cs);
}
template <int D>
__device__ inline float small_rope_q(const float* row, int c, double cs, double sn, float scale) {
#pragma clang fp contract(off)
  constexpr int H2 = D / 2;
  const int i = c < H2 ? c : c - H2;
  const double a = row[i], bb = row[i + H2];
  const float x = c < H2 ? (float)(a * cs - bb * sn) : (float)(a * sn + bb * cs);
  return x * scale;
}

// One leaf per wave; the wave's LDS holds the 16 scaled reference queries (qv,
// [16][D]) and the leaf's softmax weights (w, [16][CP]).
template <int D, int CP>
struct SmallLeaf {
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(CP == 4 || CP == 8, "padded keys");
  static constexpr int kCP = CP;                 // padded keys per leaf
  static constexpr int DPL = D / 64;             // dimensions per lane
  static constexpr int PP = 32 / CP;             // planes per pass
  static constexpr int H2 = D / 2;

  // The reference queries of head h at this lane's dimensions, rotated to
  // position pos under RoPE, scaled, into the wave's LDS.
  __device__ static void set_q(const BuildParams& P, int h, int64_t pos, float (*qv)[D], int lane) {
    const int R = P.R, d0 = DPL * lane;
    const float* qr = P.qref + (int64_t)h * R * D;
    if (!P.rope) {
      // float4 pieces, lane l taking pieces l + 64 i: every piece is loaded (a
      // padding row reads the last real row and is scaled by zero), so all the
      // loads are in flight at once instead of each waiting behind a branch on R
      constexpr int Q4 = 16 * D / 4, RQ = D / 4;
#pragma unroll
      for (int i = lane; i < Q4; i += kWave) {
        const int r = i / RQ, c = (i % RQ) * 4;
        const bool real = r < R;
        const float f = real ? P.scale : 0.0f;   // padding rows are scaled to zero
        float4 x = *(const float4*)(qr + (real ? r : R - 1) * D + c);
        x.x *= f; x.y *= f; x.z *= f; x.w *= f;
        *(float4*)&qv[r][c] = x;
      }
      wave_lds_sync();
      return;
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int c = d0 + k;
      double cs, sn;
      small_rope_angle<D>(c, pos, (double)P.rope_base, cs, sn);
#pragma unroll 2
      for (int r = 0; r < 16; ++r) {
        const int rr = r < R ? r : R - 1;
        const float x = small_rope_q<D>(qr + rr * D, c, cs, sn, P.scale);
        qv[r][d0 + k] = r < R ? x : 0.0f;
      }
    }
    wave_lds_sync();
  }

  // Leaf n of sequence-head gi, with the queries already in qv.
  typedef float Keys[CP][DPL];

  // This lane's dimensions of leaf n's keys.  A padding key (j >= C) repeats
  // the last real key: its softmax weight is zero, so any finite value serves,
  // and every load goes out at once instead of one per branch on C.
  __device__ static void load_keys(const BuildParams& P, int gi, int64_t n, Keys& kv, int lane) {
    const int C = P.C, d0 = DPL * lane;
    const uint16_t* kr = (const uint16_t*)P.K + ((int64_t)gi * P.T_cap + n * C) * D + d0;
#pragma unroll
    for (int j = 0; j < CP; ++j) {
      const int64_t row = j < C ? j : C - 1;
      if constexpr (DPL == 2) {
        const uint32_t pr = *(const uint32_t*)(kr + row * D);
        kv[j][0] = bf16_lo(pr);
        kv[j][1] = bf16_hi(pr);
      } else {
        kv[j][0] = __uint_as_float((uint32_t)kr[row * D] << 16);
      }
    }
  }

  // Leaf n of sequence-head gi, with the queries already in qv.
  __device__ static void leaf(const BuildParams& P, int gi, int64_t n, const float (*qv)[D],
                              float (*wsh)[CP], int lane) {
    Keys kv;
    load_keys(P, gi, n, kv, lane);
    leaf_from(P, gi, n, kv, qv, wsh, lane);
  }

  // Leaf n of sequence-head gi from its keys kv.
  __device__ static void leaf_from(const BuildParams& P, int gi, int64_t n, const Keys& kv,
                                   const float (*qv)[D], float (*wsh)[CP], int lane) {
    const int C = P.C, R = P.R, d0 = DPL * lane;
    // after a pass's butterfly: entry e = lane / 2, plane PP pass + e / CP, key e % CP
    const int e = lane >> 1, jl = e % CP, rl = e / CP;
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
      if ((lane & 1) == 0) wsh[r][jl] = ex / S;
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
          const float w = wsh[rr][j];            // the same address in every lane
#pragma unroll
          for (int k = 0; k < DPL; ++k) acc[k] = fmaf(w, kv[j][k], acc[k]);
        }
        if constexpr (DPL == 2) *(float2*)(kh + (int64_t)rr * D) = make_float2(acc[0], acc[1]);
        else kh[(int64_t)rr * D] = acc[0];
        if (P.khat16) {
          uint16_t* kh16 = P.khat16 + ((int64_t)gi * P.ncap + n) * R * D + d0 + (int64_t)rr * D;
          if constexpr (DPL == 2) store_bf16x2(kh16, acc[0], acc[1]);
          else kh16[0] = (uint16_t)bf16_bits(acc[0]);
        }
      }
    }
    wave_lds_sync();                       // the weights are rewritten by the next leaf
  }

  // Plane r of leaf n alone, in one wave, from its keys kv: the append's leaf,
  // with its R planes on R waves.  The arithmetic is leaf_from's, step for step
  // and in the same order (this lane's partial dots, lane sums over xor
  // distances 32 .. 1, the keys' softmax terms summed pairwise by key index
  // bits 0, 1, 2, the weights applied to the keys in key order), so the plane
  // equals the one-wave leaf's bit for bit.  Needs no LDS.
  template <bool ROPE>
  __device__ static void plane(const BuildParams& P, int gi, int h, int64_t n, int r,
                               const Keys& kv, int lane) {
    const int C = P.C, R = P.R, d0 = DPL * lane;
    const float* row = P.qref + ((int64_t)h * R + r) * D;
    float q[DPL];
    if constexpr (!ROPE) {
#pragma unroll
      for (int k = 0; k < DPL; ++k) q[k] = row[d0 + k] * P.scale;
    } else {
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        double cs, sn;
        small_rope_angle<D>(d0 + k, n * C, (double)P.rope_base, cs, sn);
        q[k] = small_rope_q<D>(row, d0 + k, cs, sn, P.scale);
      }
    }
    float z[CP];
#pragma unroll
    for (int j = 0; j < CP; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < DPL; ++k) acc = fmaf(q[k], kv[j][k], acc);
      z[j] = acc;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
      for (int j = 0; j < CP; ++j) z[j] += __shfl_xor(z[j], m, 64);
    }
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < CP; ++j) {
      if (j >= C) z[j] = -INFINITY;
      M = fmaxf(M, z[j]);
    }
    float ex[CP], s[CP], sz[CP];
#pragma unroll
    for (int j = 0; j < CP; ++j) {
      ex[j] = j < C ? expf(z[j] - M) : 0.0f;
      s[j] = ex[j];
      sz[j] = j < C ? ex[j] * z[j] : 0.0f;
    }
#pragma unroll
    for (int w = 1; w < CP; w <<= 1) {
#pragma unroll
      for (int j = 0; j < CP; j += 2 * w) {
        s[j] = s[j] + s[j + w];
        sz[j] = sz[j] + sz[j + w];
      }
    }
    const float S = s[0];
    if (lane == 0) P.bhat[((int64_t)gi * P.ncap + n) * R + r] = (M + logf(S)) - sz[0] / S;
    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = 0.0f;
#pragma unroll
    for (int j = 0; j < CP; ++j) {
      const float w = ex[j] / S;
#pragma unroll
      for (int k = 0; k < DPL; ++k) acc[k] = fmaf(w, kv[j][k], acc[k]);
    }
    float* kh = P.khat + (((int64_t)gi * P.ncap + n) * R + r) * D + d0;
    if constexpr (DPL == 2) *(float2*)kh = make_float2(acc[0], acc[1]);
    else kh[0] = acc[0];
    if (P.khat16) {
      uint16_t* kh16 = P.khat16 + (((int64_t)gi * P.ncap + n) * R + r) * D + d0;
      if constexpr (DPL == 2) store_bf16x2(kh16, acc[0], acc[1]);
      else kh16[0] = (uint16_t)bf16_bits(acc[0]);
    }
  }
};

template <int D, int CP>
__global__ void __launch_bounds__(256) build_leaves_small(BuildParams P) {
  using S = SmallLeaf<D, CP>;
  __shared__ float wsh[4][16][CP];        // per wave: the leaf's softmax weights
  __shared__ __attribute__((aligned(16))) float qsh[4][16][D];   // per wave: scaled queries
  const int gi = blockIdx.y;
  const int b = gi / P.H_kv, h = gi % P.H_kv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t n0, n1;
  node_range(P, b, n0, n1);
  if (!P.rope) S::set_q(P, h, 0, qsh[wave], lane);
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t n = n0 + (int64_t)xcd_grouped_x() * 4 + wave; n < n1; n += nw) {
    if (P.rope) S::set_q(P, h, n * P.C, qsh[wave], lane);   // (after the previous leaf's closing sync)
    S::leaf(P, gi, n, qsh[wave], wsh[wave], lane);
  }
}

// Parent summaries, one wave per (node, plane) pair: the children's planes r
// (child 4t + lane/16, dimensions (lane%16)*d/16 ..) stay in registers, and an
// exact two-pass softmax over the children gives k_hat and b_hat.  No LDS, no
// workgroup barriers.  MT: child rounds, ceil(C / 4).

// RoPE frequency of this lane, lane % (d/2) (shared with the others by shuffles).
template <int D>
__device__ inline double parent_theta(const BuildParams& P, int lane) {
  return P.rope ? pow((double)P.rope_base, -2.0 * (double)(lane % (D / 2)) / (double)D) : 0.0;
}

// The same frequency where the caller has already branched on RoPE.  The fp64
// pow is straight-line code, so the optimiser would otherwise compute it ahead
// of the branch (and out of loops) on every path; the empty asm statement on
// its input keeps it where it is written.
template <int D>
__device__ inline double rope_theta_here(float rope_base, int i) {
  asm volatile("" : "+v"(rope_base));
  return pow((double)rope_base, -2.0 * (double)i / (double)D);
}

template <int D, int MT, int RP = -1>   // RP: RoPE off (0), on (1), or P.rope (-1)
__device__ inline void parent_pair(const BuildParams& P, int gi, int h, int64_t n, int r,
                                   double theta, int lane) {
  static_assert(MT >= 1 && 4 * MT <= kMaxC, "child rounds");
  constexpr int DPL = D / 16;              // dimensions per lane
  constexpr int NV = DPL / 4;              // float4 per child per lane
  constexpr int H2 = D / 2;
  const int cg = lane >> 4, ds = (lane & 15) * DPL;
  const int C = P.C, R = P.R;
  const float* qr = P.qref + (int64_t)h * R * D;
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
  if (RP == 0 || (RP < 0 && !P.rope)) {
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
    for (int q = 0; q < NV; ++q) {
      const float4 v = make_float4(ka[4 * q] / S, ka[4 * q + 1] / S, ka[4 * q + 2] / S, ka[4 * q + 3] / S);
      *(float4*)(kh + 4 * q) = v;
      if (P.khat16)
        store_bf16x4(P.khat16 + (((int64_t)gi * P.ncap + n) * R + r) * D + ds + 4 * q, v.x, v.y, v.z, v.w);
    }
  }
  // b_hat = F - sum_j w_j z_j with F = M + log S and z_j = scale q.k_hat_{r,j}
  if (lane == 0) P.bhat[((int64_t)gi * P.ncap + n) * R + r] = (M + logf(S)) - SW / S;
}

template <int D, int MT>
__global__ void __launch_bounds__(256) build_parents(BuildParams P) {
  const int gi = blockIdx.y;
  const int b = gi / P.H_kv, h = gi % P.H_kv;
  const int lane = threadIdx.x & 63;
  const int R = P.R;
  int64_t n0, n1;
  node_range(P, b, n0, n1);
  const double theta = parent_theta<D>(P, lane);
  const int64_t npairs = (n1 - n0) * R;
  // the 32 pairs of one line of b-hat run in 8 workgroups on one XCD
  for (int64_t pr = (int64_t)xcd_grouped_x() * 4 + (threadIdx.x >> 6); pr < npairs;
       pr += (int64_t)gridDim.x * 4)
    parent_pair<D, MT>(P, gi, h, n0 + pr / R, (int)(pr % R), theta, lane);
}

// ---------------------------------------------------------------- one-launch append
//
// A decode step completes at most one chunk, so one append builds at most one
// node per level and tree: a leaf every C steps, a level-2 node every C^2, and
// so on ([ZHA] "무엇과 다른가", append cadence).  This kernel does the cascade of
// one (sequence, KV head) tree in one workgroup: its new leaves (one wave per
// leaf with the prefill's matrix-core code for C >= 16; for C <= 8 one wave per
// plane, with the prefill's arithmetic in the prefill's order; either way the
// summaries are bit for bit the prefill's), then level by level the new
// parents' (node, plane) pairs over all waves, with a workgroup barrier between
// levels (a parent reads children this workgroup has just written).  The sequence's node counts are
// shared by its H_kv trees: every workgroup reads them first thing, then
// arrives at a counter in the workspace, and the last to arrive (which returns
// the counter to zero) writes the new counts.  It loops over however many nodes
// are missing, so any growth is built, only slower.

struct AppendParams {
  int32_t L;                   // first, so the prologue's arguments share few cache lines
  int32_t* arrive;             // [B] arrival counters, zero between calls
  BuildParams lv[ZHA_MAX_L];   // level l at index l-1 (append mode)
};

constexpr int kLeafGeneric = 0, kLeafMfma = 1, kLeafSmall = 2;

// Global writes of every wave of the workgroup visible to every wave.
__device__ inline void workgroup_sync_global() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Nodes [n0, n1) of level l are missing: from the count before the call (old)
// to the count the length T completes, within the level's capacity.
__device__ inline void missing_nodes(const BuildParams& P, int l, int64_t old, int64_t T,
                                     int cshift, int64_t& n0, int64_t& n1) {
  n1 = T >> (l * cshift);
  if (n1 > P.ncap) n1 = P.ncap;
  n0 = old < 0 ? 0 : old;
  if (n0 > n1) n0 = n1;
}

// The append's parents, levels 2..L with new nodes (bit l of work): their
// (node, plane) pairs over all waves, a barrier before each level that reads
// nodes written in this launch.  RP as for parent_pair: a compile-time RoPE
// choice leaves the non-RoPE cascade without the fp64 angle code (used where
// the registers allow both copies).
template <int D, int MT, int NW, int RP>
__device__ inline void append_parents(const AppendParams& A, const int64_t* s_old, int64_t T,
                                      int cshift, uint32_t work, bool dirty, int gi, int h,
                                      int wave, int lane) {
  const int R = A.lv[0].R;
  double theta = 0.0;
  if (RP == 1 || (RP < 0 && A.lv[0].rope))
    theta = rope_theta_here<D>(A.lv[0].rope_base, lane % (D / 2));
  for (int l = 2; l <= A.L; ++l) {
    if (!((work >> l) & 1u)) continue;
    const BuildParams& P = A.lv[l - 1];
    int64_t n0, n1;
    missing_nodes(P, l, s_old[l - 1], T, cshift, n0, n1);
    if (dirty) workgroup_sync_global();
    const int64_t items = (n1 - n0) * R;
    for (int64_t i = wave; i < items; i += NW)
      parent_pair<D, MT, RP>(P, gi, h, n0 + i / R, (int)(i % R), theta, lane);
    dirty = true;
  }
}

// Plane r of every new small-C leaf of the tree on wave r (R <= 16 <= waves).
template <int D, int CL, int NW, bool ROPE>
__device__ inline void append_small_leaves(const BuildParams& P, int gi, int h, int64_t n0,
                                           int64_t n1, int wave, int lane) {
  using S = SmallLeaf<D, CL>;
  for (int64_t n = n0; n < n1; ++n)
    for (int r = wave; r < P.R; r += NW) {
      typename S::Keys kv;
      S::load_keys(P, gi, n, kv, lane);
      S::template plane<ROPE>(P, gi, h, n, r, kv, lane);
    }
}

template <int D, int KIND, int CL, int MT, int NT>
__global__ void __launch_bounds__(NT) append_chunk(AppendParams A) {
  constexpr int NW = NT / kWave;
  static_assert(KIND != kLeafGeneric || NT == kGenericThreads, "generic leaves: one workgroup");
  static_assert(KIND != kLeafSmall || NW >= 16, "small leaves: a wave per plane");
  const int gi = blockIdx.x;
  const BuildParams& P1 = A.lv[0];
  // The arguments the prologue needs, loaded together: a kernel argument first
  // read inside a branch costs a round trip of its own, and they add up.
  const int H = P1.H_kv, L = A.L, Bn = P1.B, C1 = P1.C;
  const int64_t* const Tp = P1.T;
  int64_t* const nb = P1.n_built;
  const int64_t Tcap = P1.T_cap;
  asm volatile("" ::"s"(H), "s"(L), "s"(Bn), "s"(C1), "s"(Tp), "s"(nb), "s"(Tcap));
  const int b = gi / H, h = gi % H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int last = NW - 1;   // reads the old counts and arrives
  // ---- the old node counts of every level and the length, in one round trip
  // by the last wave, while the matrix-core leaf wave stages the reference
  // queries (without RoPE they do not depend on the node)
  __shared__ int64_t s_old[ZHA_MAX_L + 1];
  if (wave == last && (lane < L || lane == kWave - 1)) {
    // one load instruction: lanes below L read a level's count, the top lane T
    const int64_t* src = lane < L ? nb + (int64_t)lane * Bn + b : Tp + b;
    s_old[lane < L ? lane : ZHA_MAX_L] = *src;
  }
  using M = MfmaLeaf<D, KIND == kLeafMfma ? CL : 16>;
  __shared__ __attribute__((aligned(16))) unsigned char leaf_lds[KIND == kLeafMfma ? M::kLds : 16];
  typename M::QOps qa;
  if constexpr (KIND == kLeafMfma) {
    if (wave == 0) {
      M::init(leaf_lds, lane);
      if (!P1.rope) M::build_qa(P1, h, 1.0, 0.0, leaf_lds, qa, lane);
    }
  }
  __syncthreads();
  int64_t T = s_old[ZHA_MAX_L];
  if (T < 0) T = 0;
  if (T > Tcap) T = Tcap;
  const int cshift = __builtin_ctz((unsigned)C1);   // C is a power of two: T / C^l by shifts
  // Which levels above the leaves have new nodes (bit l), from the length and
  // the old counts alone: a level's capacity is at least T_cap / C^l (checked
  // on the host), so it cannot cut the range here.  A leaf-only append then
  // runs no parent code and reads no parent level's arguments.
  uint32_t work = 0;
#pragma unroll
  for (int l = 2; l <= ZHA_MAX_L; ++l) {
    const int64_t old = s_old[l - 1];   // (every entry is read: no branch per level)
    work |= (uint32_t)((l <= L) & ((T >> (l * cshift)) > (old < 0 ? 0 : old))) << l;
  }
  // The sequence's node counts: every tree of it has read the old ones before
  // it arrives, so the last to arrive may write the new ones.
  auto arrive = [&] {
    const int prev = __hip_atomic_fetch_add(&A.arrive[b], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == H - 1) {
      for (int l = 1; l <= L; ++l) nb[(int64_t)(l - 1) * Bn + b] = T >> (l * cshift);
      __hip_atomic_store(&A.arrive[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  if (KIND != kLeafGeneric && threadIdx.x == last * kWave) arrive();
  // ---- level 1: the tree's new leaves: one wave each (matrix cores), one wave
  // per plane (small C), or the workgroup (generic)
  int64_t n0, n1;
  missing_nodes(P1, 1, s_old[0], T, cshift, n0, n1);
  const bool dirty = n1 > n0;   // nodes written since the last barrier
  if constexpr (KIND == kLeafGeneric) {
    __shared__ BuildSmem sm;
    for (int64_t n = n0; n < n1; ++n) generic_leaf(P1, sm, gi, h, n);
  } else if constexpr (KIND == kLeafMfma) {
    if (wave == 0 && n0 < n1) {
      double theta = 0.0;
      if (P1.rope) theta = rope_theta_here<D>(P1.rope_base, lane % M::H2);
      for (int64_t n = n0; n < n1; ++n) {
        typename M::Keys kv;
        M::fetch(P1, gi, n, kv, lane);        // in flight while the queries are staged
        if (P1.rope) {
          double cs, sn;
          sincos((double)(n * CL) * theta, &sn, &cs);
          M::build_qa(P1, h, cs, sn, leaf_lds, qa, lane);
        }
        M::leaf(P1, gi, n, kv, qa, leaf_lds, lane, [] {});
      }
    }
  } else {
    if (P1.rope) append_small_leaves<D, CL, NW, true>(P1, gi, h, n0, n1, wave, lane);
    else append_small_leaves<D, CL, NW, false>(P1, gi, h, n0, n1, wave, lane);
  }
  // ---- levels 2..L with new nodes
  if (work != 0) {
    if constexpr (KIND == kLeafSmall) {
      if (P1.rope) append_parents<D, MT, NW, 1>(A, s_old, T, cshift, work, dirty, gi, h, wave, lane);
      else append_parents<D, MT, NW, 0>(A, s_old, T, cshift, work, dirty, gi, h, wave, lane);
    } else {
      append_parents<D, MT, NW, -1>(A, s_old, T, cshift, work, dirty, gi, h, wave, lane);
    }
  }
  if (KIND == kLeafGeneric && threadIdx.x == 0) arrive();
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
  P.khat16 = tree->khat16[level - 1];
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

// The one-launch append: one workgroup per (sequence, KV head).  Leaves take the
// prefill's kernel family for the geometry; parents take ceil(C / 4) child
// rounds (the workgroup size follows their registers).
template <int D>
static void launch_append_d(const AppendParams& A, hipStream_t s) {
  const BuildParams& P = A.lv[0];
  const dim3 grid((unsigned)(P.B * P.H_kv));
  const bool bf = P.kv_dtype == ZHA_BF16 && P.R <= 16;
  if (bf && P.C == 64) hipLaunchKernelGGL((append_chunk<D, kLeafMfma, 64, 16, 512>), grid, dim3(512), 0, s, A);
  else if (bf && P.C == 32) hipLaunchKernelGGL((append_chunk<D, kLeafMfma, 32, 8, 512>), grid, dim3(512), 0, s, A);
  else if (bf && P.C == 16) hipLaunchKernelGGL((append_chunk<D, kLeafMfma, 16, 4, 512>), grid, dim3(512), 0, s, A);
  else if (bf && P.C == 8) hipLaunchKernelGGL((append_chunk<D, kLeafSmall, 8, 2, 1024>), grid, dim3(1024), 0, s, A);
  else if (bf) hipLaunchKernelGGL((append_chunk<D, kLeafSmall, 4, 1, 1024>), grid, dim3(1024), 0, s, A);
  else if (P.C <= 4) hipLaunchKernelGGL((append_chunk<D, kLeafGeneric, 0, 1, kGenericThreads>), grid, dim3(kGenericThreads), 0, s, A);
  else if (P.C == 8) hipLaunchKernelGGL((append_chunk<D, kLeafGeneric, 0, 2, kGenericThreads>), grid, dim3(kGenericThreads), 0, s, A);
  else if (P.C == 16) hipLaunchKernelGGL((append_chunk<D, kLeafGeneric, 0, 4, kGenericThreads>), grid, dim3(kGenericThreads), 0, s, A);
  else if (P.C == 32) hipLaunchKernelGGL((append_chunk<D, kLeafGeneric, 0, 8, kGenericThreads>), grid, dim3(kGenericThreads), 0, s, A);
  else hipLaunchKernelGGL((append_chunk<D, kLeafGeneric, 0, 16, kGenericThreads>), grid, dim3(kGenericThreads), 0, s, A);
}

static void launch_append_chunk(const AppendParams& A, hipStream_t s) {
  if (A.lv[0].d == 128) launch_append_d<128>(A, s);
  else launch_append_d<64>(A, s);
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
  rc = zha_check_ws(cfg, ZHA_OP_BUILD, ws, ws_bytes);
  if (rc != ZHA_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (max_new_tokens <= cfg->C) {
    // at most one new node per level and tree: the one-launch cascade
    zha::AppendParams A;
    for (int level = 1; level <= cfg->L; ++level)
      A.lv[level - 1] = zha::make_params(cfg, kv, qref, tree, level, 1);
    A.L = cfg->L;
    A.arrive = (int32_t*)((char*)ws + zha::ws_layout(*cfg).build_off);
    zha::launch_append_chunk(A, s);
    return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_EHIP;
  }
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
