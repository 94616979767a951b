// libsla host entry points that launch nothing: version, status names, block counts,
// capacities and workspace sizes.
#include "sla_host.h"

extern "C" {

int32_t sla_abi_version(void) { return SLA_ABI_VERSION; }

const char* sla_status_str(sla_status s) {
  switch (s) {
    case SLA_OK: return "ok";
    case SLA_ERR_NULL: return "required pointer is NULL";
    case SLA_ERR_SHAPE: return "inconsistent or unsupported sizes";
    case SLA_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case SLA_ERR_RANGE: return "count, share or length out of range";
    case SLA_ERR_UNSUPPORTED: return "unsupported combination";
    case SLA_ERR_CAPACITY: return "output capacity too small";
    case SLA_ERR_HIP: return "HIP launch failed";
    case SLA_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

sla_status sla_counts(int32_t nb, int32_t kh_bp, int32_t kl_bp, int32_t* n_crit, int32_t* n_negl) {
  if (n_crit == nullptr || n_negl == nullptr) return SLA_ERR_NULL;
  if (nb < 1 || kh_bp < 0 || kh_bp > 10000 || kl_bp < 0 || kl_bp > 10000) return SLA_ERR_RANGE;
  const int64_t nh = kh_bp == 0 ? 0 : (int64_t(kh_bp) * nb + 9999) / 10000;
  const int64_t h = nh < nb ? nh : nb;
  const int64_t nl = int64_t(kl_bp) * nb / 10000;
  *n_crit = int32_t(h);
  *n_negl = int32_t(nl < nb - h ? nl : nb - h);
  return SLA_OK;
}

int64_t sla_block_map_capacity(int32_t B, int32_t Hs, int32_t nqb, int32_t nkb, int32_t n_crit,
                               int32_t n_negl, int32_t causal, int32_t window_tokens, int32_t which) {
  if (B < 1 || Hs < 1 || nqb < 1 || nkb < 1 || n_crit < 0 || n_negl < 0 || window_tokens < 0) return -1;
  const int64_t rows = int64_t(B) * Hs * nqb;
  if (!causal) {
    if (n_crit + n_negl > nkb) return -1;
    return which == 0 ? rows * n_crit : rows * (nkb - n_crit - n_negl);
  }
  if (nqb != nkb) return -1;
  if (which != 0) return 0;
  const int32_t reach = sla::window_reach(window_tokens);
  int64_t per_head = 0;
  for (int32_t i = 0; i < nqb; ++i) {
    int64_t c = int64_t(n_crit) + reach + 1;
    if (c > i + 1) c = i + 1;
    per_head += c;
  }
  return per_head * B * Hs;
}

size_t sla_block_map_workspace_bytes(int32_t B, int32_t Hs, int32_t nqb, int32_t nkb, int32_t n_crit,
                                     int32_t causal, int32_t window_tokens) {
  if (!causal || B < 1 || Hs < 1 || nqb < 1) return 0;
  (void)nkb;
  const int64_t row_cap = int64_t(n_crit) + sla::window_reach(window_tokens) + 1;
  const int64_t rows = int64_t(B) * Hs * nqb;
  // padded per-row block lists (int32) + flags (uint8), each 256-byte aligned
  const int64_t idx = (rows * row_cap * 4 + 255) / 256 * 256;
  const int64_t fl = (rows * row_cap + 255) / 256 * 256;
  return size_t(idx + fl);
}

size_t sla_kv_reduce_workspace_bytes(int32_t B, int32_t Hkv, int32_t N, int32_t d, int32_t want_blocks,
                                     int32_t want_all) {
  (void)want_blocks;   // per-block states need no workspace; the sum over all keys does
  if (!want_all || B < 1 || Hkv < 1 || N < SLA_BLOCK) return 0;
  const int64_t nb = N / SLA_BLOCK;
  const int run = sla::kv_sum_run(nb, int64_t(B) * Hkv);
  const int64_t chunks = (nb + run - 1) / run;   // fp32 partial state per run
  return size_t(int64_t(B) * Hkv * chunks * (int64_t(d) * d + d) * 4);
}

size_t sla_attn_workspace_bytes(int32_t B, int32_t Hs, int32_t nqb, int32_t d, int32_t lin_mode) {
  if (lin_mode != SLA_LIN_MARGINAL || B < 1 || Hs < 1 || nqb < 1) return 0;
  const int64_t rows = int64_t(B) * Hs * nqb;
  return size_t(rows * (int64_t(d) * d * 2 + int64_t(d) * 4));   // bf16 row sums + fp32 u
}

}  // extern "C"
