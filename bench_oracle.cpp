// bench_oracle.cpp -- times the CPU oracle (oracle/pero.c) on a workload's
// steps for the CPU-baseline figure of bench.py ("Putting prioritized
// replay's segment tree on a GPU", section "Measuring the Trade Honestly":
// the same operations timed on the CPU next to the GPU).
//
// The oracle is called exactly as it stands, one thread, one call per
// operation; only the clock around the calls lives here.  Each call is timed
// with std::chrono::steady_clock, so that no interpreter or argument
// marshalling is counted.  The initial fill is not timed.
//
// Built by bench.build_oracle_timer() together with a copy of pero.c
// compiled with the oracle's own flags.

#include <chrono>
#include <cstdint>
#include <vector>

#include "oracle/pero.h"

namespace {

using Clock = std::chrono::steady_clock;

double seconds_since(Clock::time_point t0) {
  return std::chrono::duration<double>(Clock::now() - t0).count();
}

}  // namespace

extern "C" {

// Creates an oracle of capacity n (state_dim D, alpha, eps), fills it with
// n items (priorities prio, or the running max when NULL; rows when D > 0),
// then runs steps of
//   sample(B masses u) -> update(idx or the sampled slots, td) -> add(intake)
// with step s taking u[s * B ...], td[s * B ...] and idx[s * B ...] (idx may
// be NULL), s cycling over nsteps, until max_steps steps have run or the
// timed CPU time passes max_seconds.  Samples take IS weights when weights
// != 0 and gather rows when rows != 0.  out[0..2]: seconds spent in sample,
// update and add; out[3]: steps run.  Returns 0, or -1 if the oracle
// refused the workload.
int oracle_time_steps(int64_t n, int32_t D, double alpha, double eps, const float* prio,
                      const float* states, const float* next_states, const uint32_t* actions,
                      const float* rewards, const uint8_t* dones, int64_t B, int64_t nsteps,
                      const float* u, const float* td, const int64_t* idx, int64_t intake,
                      double beta, int32_t weights, int32_t rows, int64_t max_steps,
                      double max_seconds, double* out) {
  pero_t* t = pero_create(n, D, alpha, eps);
  if (!t) return -1;
  if (pero_add(t, n, states, next_states, actions, rewards, dones, prio) != 0) {
    pero_destroy(t);
    return -1;
  }
  std::vector<int64_t> sidx(B);
  std::vector<float> w(weights ? B : 0);
  const bool gather = rows && D > 0;
  std::vector<float> s_out(gather ? B * D : 0), n_out(gather ? B * D : 0);
  std::vector<float> r_out(gather ? B : 0);
  std::vector<uint32_t> a_out(gather ? B : 0);
  std::vector<uint8_t> d_out(gather ? B : 0);
  // intake rows (when the oracle keeps rows): the first `intake` stored rows
  const bool intake_rows = D > 0 && intake > 0 && states;
  double ts = 0.0, tu = 0.0, ta = 0.0;
  int64_t done = 0;
  int rc = 0;
  while (done < max_steps && ts + tu + ta < max_seconds) {
    const int64_t s = done % nsteps;
    Clock::time_point t0 = Clock::now();
    rc = pero_sample(t, B, u + s * B, beta, sidx.data(), weights ? w.data() : nullptr,
                     gather ? s_out.data() : nullptr, gather ? n_out.data() : nullptr,
                     gather ? a_out.data() : nullptr, gather ? r_out.data() : nullptr,
                     gather ? d_out.data() : nullptr);
    ts += seconds_since(t0);
    if (rc != 0) break;
    const int64_t* ui = idx ? idx + s * B : sidx.data();
    t0 = Clock::now();
    rc = pero_update(t, B, ui, td + s * B);
    tu += seconds_since(t0);
    if (rc != 0) break;
    if (intake > 0) {
      t0 = Clock::now();
      rc = pero_add(t, intake, intake_rows ? states : nullptr, intake_rows ? next_states : nullptr,
                    intake_rows ? actions : nullptr, intake_rows ? rewards : nullptr,
                    intake_rows ? dones : nullptr, nullptr);
      ta += seconds_since(t0);
      if (rc != 0) break;
    }
    ++done;
  }
  pero_destroy(t);
  out[0] = ts;
  out[1] = tu;
  out[2] = ta;
  out[3] = (double)done;
  return rc == 0 ? 0 : -1;
}

}  // extern "C"
