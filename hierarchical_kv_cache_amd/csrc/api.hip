// Host-side argument checks, workspace sizing and status helpers of libzha.
#include "zha_internal.hpp"

#include <math.h>

extern "C" size_t zha_workspace_bytes(const zha_cfg* cfg, int32_t op) {
  if (cfg == nullptr || zha_check_cfg(cfg) != ZHA_OK) return 0;
  zha::WsLayout w = zha::ws_layout(*cfg);
  switch (op) {
    case ZHA_OP_BUILD: return w.build_off + w.build_bytes;
    case ZHA_OP_ROUTE: return w.route_off + w.route_bytes;
    case ZHA_OP_ATTEND:
    case ZHA_OP_DENSE:
    case ZHA_OP_ALL: return w.total;
    default: return 0;
  }
}

extern "C" const char* zha_status_str(int32_t s) {
  switch (s) {
    case ZHA_OK: return "ZHA_OK";
    case ZHA_EINVAL: return "ZHA_EINVAL: invalid argument";
    case ZHA_EUNSUPPORTED: return "ZHA_EUNSUPPORTED: unsupported geometry or dtype";
    case ZHA_EWORKSPACE: return "ZHA_EWORKSPACE: workspace too small or null";
    case ZHA_ECAPACITY: return "ZHA_ECAPACITY: list capacity exceeded";
    case ZHA_EHIP: return "ZHA_EHIP: HIP runtime error";
    case ZHA_ESTALE: return "ZHA_ESTALE: tree does not match T";
    default: return "ZHA: unknown status";
  }
}

int32_t zha_check_cfg(const zha_cfg* c) {
  if (c == nullptr) return ZHA_EINVAL;
  if (c->B < 1 || c->H_kv < 1 || c->G < 1 || c->L < 1 || c->R < 1 || c->C < 1)
    return ZHA_EINVAL;
  if (c->T_cap < 1 || c->leaf_cap < 0) return ZHA_EINVAL;
  if (!(c->scale > 0.0f) || !isfinite(c->scale)) return ZHA_EINVAL;
  if (c->L > ZHA_MAX_L) return ZHA_EUNSUPPORTED;
  if (c->G > ZHA_MAX_G) return ZHA_EUNSUPPORTED;
  if (c->R > 16) return ZHA_EUNSUPPORTED;
  if (c->d != 64 && c->d != 128) return ZHA_EUNSUPPORTED;
  if (c->C < 2 || c->C > 64 || (c->C & (c->C - 1)) != 0) return ZHA_EUNSUPPORTED;
  if (c->kv_dtype != ZHA_F32 && c->kv_dtype != ZHA_BF16) return ZHA_EUNSUPPORTED;
  if (c->rope != 0 && c->rope != 1) return ZHA_EINVAL;
  if (c->rope == 1 && !(c->rope_base > 1.0f)) return ZHA_EINVAL;
  // ids are int32: every level's node count and the token count must fit
  if (c->T_cap > (int64_t)INT32_MAX) return ZHA_EUNSUPPORTED;
  return ZHA_OK;
}

int32_t zha_check_ws(const zha_cfg* cfg, int32_t op, const void* ws, size_t ws_bytes) {
  size_t need = zha_workspace_bytes(cfg, op);
  if (need == 0) return ZHA_EINVAL;
  if (ws == nullptr || ws_bytes < need) return ZHA_EWORKSPACE;
  if (((uintptr_t)ws & 255) != 0) return ZHA_EWORKSPACE;
  return ZHA_OK;
}

extern "C" int32_t zha_ws_status(void* ws, void* stream, int32_t* status) {
  if (ws == nullptr || status == nullptr) return ZHA_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  int32_t host = 0;
  if (hipMemcpyAsync(&host, ws, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
    return ZHA_EHIP;
  if (hipMemsetAsync(ws, 0, sizeof(int32_t), s) != hipSuccess) return ZHA_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return ZHA_EHIP;
  *status = host;
  return ZHA_OK;
}

// Per-level top-p of a depth schedule, computed in double and rounded once to
// float.  The weights of the power schedule are l^-gamma normalised to sum to
// one, so the product of the levels' p is p itself.
extern "C" int32_t zha_p_schedule(int32_t kind, float p, int32_t L, float gamma, float* p_levels) {
  if (p_levels == nullptr || L < 1 || L > ZHA_MAX_L) return ZHA_EINVAL;
  if (!(p > 0.0f) || !(p <= 1.0f)) return ZHA_EINVAL;
  const double lp = log((double)p);
  switch (kind) {
    case ZHA_SCHED_UNIFORM:
      for (int l = 0; l < L; ++l) p_levels[l] = p;
      return ZHA_OK;
    case ZHA_SCHED_ROOT:
      for (int l = 0; l < L; ++l) p_levels[l] = (float)exp(lp / (double)L);
      return ZHA_OK;
    case ZHA_SCHED_POWER: {
      if (!isfinite(gamma)) return ZHA_EINVAL;
      double tot = 0.0;
      for (int l = 1; l <= L; ++l) tot += pow((double)l, -(double)gamma);
      for (int l = 1; l <= L; ++l) p_levels[l - 1] = (float)exp(lp * pow((double)l, -(double)gamma) / tot);
      return ZHA_OK;
    }
    default:
      return ZHA_EINVAL;
  }
}
