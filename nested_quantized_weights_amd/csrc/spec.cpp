// Choosing the draft length k ("How Speculative Decoding Speeds Up
// Inference", section "Tokens per pass and time per token"): expected tokens
// per pass (Eq. (1)), time per token (Eq. (2)) from measured draft and pass
// times, the k with the least time per token, and a running acceptance rate
// from the rounds seen so far. Host code: every pointer here is a host
// pointer, and nothing touches the GPU.
#include <cmath>

#include "common.h"

extern "C" double nest_expected_tokens(double alpha, int64_t k) {
  if (!(alpha >= 0.0 && alpha <= 1.0) || k < 0) {
    nest::fail(NEST_EINVAL, "nest_expected_tokens: need 0 <= alpha <= 1 and k >= 0");
    return NAN;
  }
  // 1 + a + a^2 + ... + a^k: slot j is reached with probability a^j when
  // every slot is accepted independently with probability a.
  double e = 1.0;
  for (int64_t j = 0; j < k; ++j) e = 1.0 + alpha * e;
  return e;
}

extern "C" double nest_token_time(double alpha, int64_t k, double t_draft, double t_pass) {
  const double e = nest_expected_tokens(alpha, k);
  if (std::isnan(e)) return NAN;
  return (t_pass + static_cast<double>(k) * t_draft) / e;
}

extern "C" int64_t nest_choose_k(double alpha, double t_draft, const double* t_pass, int64_t kmax,
                                 double* t_token) {
  if (!t_pass || kmax < 0 || !(alpha >= 0.0 && alpha <= 1.0) || !(t_draft >= 0.0)) {
    nest::fail(NEST_EINVAL, "nest_choose_k: need t_pass, kmax >= 0, 0 <= alpha <= 1, t_draft >= 0");
    return -1;
  }
  int64_t best = 0;
  double tb = nest_token_time(alpha, 0, t_draft, t_pass[0]);
  for (int64_t k = 1; k <= kmax; ++k) {
    const double t = nest_token_time(alpha, k, t_draft, t_pass[k]);
    if (t < tb) {  // strictly better: ties keep the shorter draft
      tb = t;
      best = k;
    }
  }
  if (t_token) *t_token = tb;
  nest::ok();
  return best;
}

extern "C" void nest_alpha_init(nest_alpha* st, double decay, double prior_accepted, double prior_rejected) {
  if (!st) return;
  st->decay = decay;
  st->accepted = prior_accepted;
  st->rejected = prior_rejected;
}

extern "C" void nest_alpha_update(nest_alpha* st, int64_t accepted, int64_t k) {
  if (!st) return;
  // a round that kept `accepted` of k drafts judged accepted + (accepted < k)
  // slots: the accepted ones and, unless all k were kept, one rejected slot
  st->accepted = st->decay * st->accepted + static_cast<double>(accepted);
  st->rejected = st->decay * st->rejected + (accepted < k ? 1.0 : 0.0);
}

extern "C" double nest_alpha_value(const nest_alpha* st) {
  if (!st) return NAN;
  const double n = st->accepted + st->rejected;
  return n > 0.0 ? st->accepted / n : 0.0;
}
