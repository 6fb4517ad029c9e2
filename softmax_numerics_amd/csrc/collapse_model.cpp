// Closed forms of the P-cast collapse model, for predicting at run time whether a
// configuration will zero the non-sink probabilities.
//
// Model (P-cast summary on gist.science, section "Metodologia e Analisi"): in
// natural-log logit units the non-sink logits are i.i.d. N(0,1) and k sink keys
// carry z + Delta.  Under forward order the running max that every later
// non-sink key is taken relative to is about the largest sink logit, Delta + M_k
// with M_k the max of k standard normals.  A non-sink probability exp(z - Delta -
// M_k) gets the E4M3 code 0 when S times it is at most 2^-10, i.e. when
// z <= Delta + M_k - 10 ln 2 - ln S.  Hence, with Phi the normal CDF:
//
//   underflow fraction      F*(Delta, S) = E[Phi(Delta + M_k - 10 ln 2 - ln S)]
//   lost non-sink mass      E[Phi(Delta + M_k - 10 ln 2 - ln S - 1)]
//       (the mass weights exp(z) shift the normal density by one:
//        exp(z) phi(z) = exp(1/2) phi(z - 1))
//   collapse threshold      Delta_c(S) = 10 ln 2 + ln S - E[M_k]
//       (where the summary's plug-in form Phi(Delta + E[M_k] - 10 ln 2 - ln S)
//        crosses 1/2; section "Contributi Chiave", point 1)
//
// Expectations over M_k are integrals against its density k phi(x) Phi(x)^(k-1),
// by composite Simpson's rule on [-12, 12] (the density is below 1e-30 outside).
#include <cmath>

#include "pcast_attn.h"

namespace {

constexpr double kPi = 3.14159265358979323846;

double normal_pdf(double x) { return std::exp(-0.5 * x * x) / std::sqrt(2.0 * kPi); }
double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }
double max_pdf(double x, int k) { return k * normal_pdf(x) * std::pow(normal_cdf(x), k - 1); }

template <class F>
double expect_max(int k, F f) {
  const int n = 24000;  // even
  const double a = -12.0, h = 24.0 / n;
  double sum = max_pdf(a, k) * f(a) + max_pdf(-a, k) * f(-a);
  for (int i = 1; i < n; ++i) {
    const double x = a + i * h;
    sum += (i % 2 ? 4.0 : 2.0) * max_pdf(x, k) * f(x);
  }
  return sum * h / 3.0;
}

bool bad(double S, int k) { return !(S > 0.0) || !std::isfinite(S) || k < 1 || k > 1024; }

}  // namespace

extern "C" {

double pcast_sink_max_mean(int k) {
  if (k < 1 || k > 1024) return NAN;
  return expect_max(k, [](double x) { return x; });
}

double pcast_delta_critical(double S, int k) {
  if (bad(S, k)) return NAN;
  return 10.0 * std::log(2.0) + std::log(S) - pcast_sink_max_mean(k);
}

double pcast_underflow_model(double delta, double S, int k) {
  if (bad(S, k) || !std::isfinite(delta)) return NAN;
  const double shift = delta - 10.0 * std::log(2.0) - std::log(S);
  return expect_max(k, [shift](double x) { return normal_cdf(shift + x); });
}

double pcast_lost_mass_model(double delta, double S, int k) {
  if (bad(S, k) || !std::isfinite(delta)) return NAN;
  return pcast_underflow_model(delta - 1.0, S, k);
}

int pcast_collapse_check(const float* bias, int N, double S, int order, double* delta, int* k,
                         double* delta_c, double* underflow, int* collapse) {
  if (N <= 0 || !(S > 0.0) || !std::isfinite(S) || (order != PCAST_ORDER_FORWARD && order != PCAST_ORDER_REVERSE))
    return PCAST_EINVAL;
  // the sink strength is the largest bias; the sinks are the keys that carry it
  double dmax = 0.0;
  int nk = 0;
  if (bias) {
    for (int j = 0; j < N; ++j) {
      if (!std::isfinite(bias[j])) return PCAST_EINVAL;
      if (bias[j] > dmax) {
        dmax = bias[j];
        nk = 0;
      }
      if (bias[j] == dmax && dmax > 0.0) ++nk;
    }
  }
  const bool sinks = nk > 0 && nk <= 1024;
  const double dc = sinks ? pcast_delta_critical(S, nk) : NAN;
  const double f = sinks ? pcast_underflow_model(dmax, S, nk) : 0.0;
  if (delta) *delta = dmax;
  if (k) *k = nk;
  if (delta_c) *delta_c = dc;
  if (underflow) *underflow = f;
  if (collapse) *collapse = (sinks && order == PCAST_ORDER_FORWARD && dmax > dc) ? 1 : 0;
  return PCAST_OK;
}

}  // extern "C"
