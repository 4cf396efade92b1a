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

// Reference queries of node n at `level`, rotated when P.rope, into qh[R][d].
__device__ inline void load_ref_queries(const BuildParams& P, int h, int64_t pos,
                                        float* qh, int ld) {
  const int d = P.d, half = d / 2;
  const float* qr = P.qref + (int64_t)h * P.R * d;
  if (!P.rope) {
    for (int idx = threadIdx.x; idx < P.R * d; idx += blockDim.x)
      qh[(idx / d) * ld + idx % d] = qr[idx];
    return;
  }
  for (int idx = threadIdx.x; idx < P.R * half; idx += blockDim.x) {
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

__global__ void __launch_bounds__(256) build_parents(BuildParams P) {
  __shared__ BuildSmem sm;
  const int gi = blockIdx.y;
  const int b = gi / P.H_kv, h = gi % P.H_kv;
  int64_t n0, n1;
  node_range(P, b, n0, n1);
  const int d = P.d, C = P.C, R = P.R;
  for (int64_t n = n0 + blockIdx.x; n < n1; n += gridDim.x) {
    load_ref_queries(P, h, n * P.span, &sm.qh[0][0], kMaxD + 1);
    const int64_t ch0 = n * C;   // first child
    for (int r = 0; r < R; ++r) {
      // children's plane r -> LDS
      for (int idx = threadIdx.x; idx < C * d; idx += blockDim.x) {
        const int j = idx / d, c = idx % d;
        sm.k[j][c] = P.khat_ch[(((int64_t)gi * P.ncap_ch + ch0 + j) * R + r) * d + c];
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
  if (P.level == 1)
    hipLaunchKernelGGL(build_leaves, grid, dim3(256), 0, s, P);
  else
    hipLaunchKernelGGL(build_parents, grid, dim3(256), 0, s, P);
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
