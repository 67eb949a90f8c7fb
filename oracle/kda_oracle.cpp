// FP64 CPU oracle for the Kimi Delta Attention (KDA) training path.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
// this file; it exists so that the GPU library can be checked against a plain
// definition. It shares no code with the GPU kernels.
//
// What it computes (per head h, per packed document [cu[d], cu[d+1])):
//   gated delta rule with a per-channel (diagonal) forget gate, as described on
//   flashinfer PR #8909 ("fix(cake_kda_det): gate-gradient accuracy of the GLM
//   intra stage"), opening section: the deterministic single-device KDA
//   training package with gate form g or raw, optional fused Q/K L2 norm and a
//   saved or replay backward; documents packed into one sequence are described
//   in the opening section of flashinfer PR #7176 ("perf(cake_kda): ... BF16x3
//   half-width transfer walk"). The pages print no equations; the recurrence
//   written out below is the plain reading of the gated delta rule that the
//   chunked form (per-chunk affine state map S_out = M*S_in + B, PR #7176
//   opening section) is an acceleration of:
//
//     S_0 = 0 at every document start, except that document 0 may enter with a
//         given state S_init (one rank's share of a sequence split over ranks,
//         PR #7176 opening section: the state passed between fragments)
//     S'_t = Diag(exp(g_t)) S_{t-1}               (decay each key row c)
//     u_t  = v_t - S'_t^T k_t
//     S_t  = S'_t + beta_t k_t u_t^T              (= (I - b k k^T) Diag(e^g) S + b k v^T)
//     o_t  = scale * S_t^T q_t
//
//   gate form "raw": g[t,h,c] = -exp(A_log[h]) * softplus(a[t,h,c] + dt_bias[h,c])
//   fused L2 norm:   q <- q * (sum_c q_c^2 + eps)^(-1/2), same for k
//
// The state after the last document may be returned as S_final, and the
// backward may take dS_final, the gradient of the loss with respect to it, and
// return dS_init, the gradient with respect to S_init.
//
// The backward is the reverse-mode derivative of the loss L = sum_t <o_t, dO_t>,
// derived by hand from the recurrence above (token by token, in reverse), with
// FP64 state checkpoints every 64 tokens and recompute inside each block.
//
// Every floating-point value is double. Build: -O2 -ffp-contract=off, no
// fast-math, no intrinsics.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

struct Problem {
  int64_t T;
  int32_t H;
  int32_t N;       // number of packed documents
  int32_t K;       // key dim (state rows)
  int32_t V;       // value dim (state columns)
  int32_t gate_raw;
  int32_t l2norm;
  double scale;
  double l2_eps;
};

struct Inputs {
  const int64_t* cu;      // [N+1]
  const double* q;        // [T,H,K]
  const double* k;        // [T,H,K]
  const double* v;        // [T,H,V]
  const double* beta;     // [T,H]
  const double* gate;     // g [T,H,K] or a [T,H,K]
  const double* A_log;    // [H]     (raw only)
  const double* dt_bias;  // [H,K]   (raw only)
};

double softplus(double x) {
  // log(1 + e^x), written so that e^x cannot overflow.
  if (x > 30.0) return x + std::log1p(std::exp(-x));
  return std::log1p(std::exp(x));
}

double sigmoid(double x) {
  if (x >= 0) return 1.0 / (1.0 + std::exp(-x));
  double e = std::exp(x);
  return e / (1.0 + e);
}

// States at the ends of the packed sequence, each [H, K, V] (nullable).
struct Boundary {
  const double* s_init;    // state entering document 0
  double* s_final;         // state leaving the last document
  const double* ds_final;  // gradient with respect to s_final
  double* ds_init;         // gradient with respect to s_init
};

// Per-token quantities of one (document, head) job, after the gate transform
// and the optional L2 norm.
struct Token {
  std::vector<double> q, k, v, g, a;  // a = exp(g)
  std::vector<double> rq, rk;         // L2 scalars (1 when L2 is off)
  std::vector<double> beta;
};

void load_job(const Problem& P, const Inputs& in, int d, int h, Token& tk) {
  const int64_t t0 = in.cu[d], t1 = in.cu[d + 1];
  const int64_t n = t1 - t0;
  const int K = P.K, V = P.V, H = P.H;
  tk.q.assign(n * K, 0);
  tk.k.assign(n * K, 0);
  tk.v.assign(n * V, 0);
  tk.g.assign(n * K, 0);
  tk.a.assign(n * K, 0);
  tk.rq.assign(n, 1.0);
  tk.rk.assign(n, 1.0);
  tk.beta.assign(n, 0);
  for (int64_t i = 0; i < n; ++i) {
    const int64_t t = t0 + i;
    const double* qs = in.q + (t * H + h) * K;
    const double* ks = in.k + (t * H + h) * K;
    const double* vs = in.v + (t * H + h) * V;
    const double* gs = in.gate + (t * H + h) * K;
    tk.beta[i] = in.beta[t * H + h];
    double sq = 0, sk = 0;
    for (int c = 0; c < K; ++c) {
      sq += qs[c] * qs[c];
      sk += ks[c] * ks[c];
    }
    if (P.l2norm) {
      tk.rq[i] = 1.0 / std::sqrt(sq + P.l2_eps);
      tk.rk[i] = 1.0 / std::sqrt(sk + P.l2_eps);
    }
    for (int c = 0; c < K; ++c) {
      tk.q[i * K + c] = qs[c] * tk.rq[i];
      tk.k[i * K + c] = ks[c] * tk.rk[i];
      double g;
      if (P.gate_raw) {
        g = -std::exp(in.A_log[h]) * softplus(gs[c] + in.dt_bias[h * K + c]);
      } else {
        g = gs[c];
      }
      tk.g[i * K + c] = g;
      tk.a[i * K + c] = std::exp(g);
    }
    for (int j = 0; j < V; ++j) tk.v[i * V + j] = vs[j];
  }
}

// One token of the forward recurrence: S (K x V, row-major) holds S_{t-1} on
// entry and S_t on exit. If Sp is given it receives S'_t, if u is given it
// receives u_t.
void step_fwd(int K, int V, const Token& tk, int64_t i, std::vector<double>& S,
              double* Sp, double* u) {
  const double* kt = &tk.k[i * K];
  const double* at = &tk.a[i * K];
  const double* vt = &tk.v[i * V];
  for (int c = 0; c < K; ++c)
    for (int j = 0; j < V; ++j) S[c * V + j] *= at[c];
  if (Sp) std::memcpy(Sp, S.data(), sizeof(double) * K * V);
  std::vector<double> ut(V);
  for (int j = 0; j < V; ++j) {
    double acc = 0;
    for (int c = 0; c < K; ++c) acc += S[c * V + j] * kt[c];
    ut[j] = vt[j] - acc;
  }
  const double b = tk.beta[i];
  for (int c = 0; c < K; ++c)
    for (int j = 0; j < V; ++j) S[c * V + j] += b * kt[c] * ut[j];
  if (u) std::memcpy(u, ut.data(), sizeof(double) * V);
}

void fwd_job(const Problem& P, const Inputs& in, const Boundary& bd, int d, int h, double* o,
             double* states, const int64_t* chunk_base, int chunk) {
  Token tk;
  load_job(P, in, d, h, tk);
  const int64_t t0 = in.cu[d];
  const int64_t n = in.cu[d + 1] - t0;
  const int K = P.K, V = P.V, H = P.H;
  std::vector<double> S(K * V, 0.0);
  if (d == 0 && bd.s_init) std::memcpy(S.data(), bd.s_init + (int64_t)h * K * V, sizeof(double) * K * V);
  for (int64_t i = 0; i < n; ++i) {
    if (states && i % chunk == 0) {
      double* dst = states + ((chunk_base[d] + i / chunk) * H + h) * K * V;
      std::memcpy(dst, S.data(), sizeof(double) * K * V);
    }
    step_fwd(K, V, tk, i, S, nullptr, nullptr);
    if (o) {
      const double* qt = &tk.q[i * K];
      double* ot = o + ((t0 + i) * H + h) * V;
      for (int j = 0; j < V; ++j) {
        double acc = 0;
        for (int c = 0; c < K; ++c) acc += S[c * V + j] * qt[c];
        ot[j] = P.scale * acc;
      }
    }
  }
  if (d == P.N - 1 && bd.s_final)
    std::memcpy(bd.s_final + (int64_t)h * K * V, S.data(), sizeof(double) * K * V);
}

struct Grads {
  double* dq;       // [T,H,K]
  double* dk;       // [T,H,K]
  double* dv;       // [T,H,V]
  double* dbeta;    // [T,H]
  double* dgate;    // dg [T,H,K] (g form) or da [T,H,K] (raw form)
  double* dA_log_part;    // [N,H]   per-job partial (raw only)
  double* ddt_bias_part;  // [N,H,K] per-job partial (raw only)
};

void bwd_job(const Problem& P, const Inputs& in, const Boundary& bd, const double* dO,
             const Grads& G, int d, int h) {
  Token tk;
  load_job(P, in, d, h, tk);
  const int64_t t0 = in.cu[d];
  const int64_t n = in.cu[d + 1] - t0;
  const int K = P.K, V = P.V, H = P.H;
  const int64_t B = 64;  // checkpoint interval
  const int64_t nblk = (n + B - 1) / B;

  // Forward pass, keeping S at the start of every block.
  std::vector<double> ckpt(nblk * K * V, 0.0);
  {
    std::vector<double> S(K * V, 0.0);
    if (d == 0 && bd.s_init) std::memcpy(S.data(), bd.s_init + (int64_t)h * K * V, sizeof(double) * K * V);
    for (int64_t i = 0; i < n; ++i) {
      if (i % B == 0) std::memcpy(&ckpt[(i / B) * K * V], S.data(), sizeof(double) * K * V);
      step_fwd(K, V, tk, i, S, nullptr, nullptr);
    }
  }

  // gradient w.r.t. S_t; zero after a document, dS_final after the last one
  std::vector<double> dS(K * V, 0.0);
  if (d == P.N - 1 && bd.ds_final)
    std::memcpy(dS.data(), bd.ds_final + (int64_t)h * K * V, sizeof(double) * K * V);
  std::vector<double> Sp_blk(B * K * V), St_blk(B * K * V), u_blk(B * V);
  std::vector<double> dqh(n * K, 0.0), dkh(n * K, 0.0), dg(n * K, 0.0);
  std::vector<double> du(V), dSp(K * V);

  for (int64_t b = nblk - 1; b >= 0; --b) {
    const int64_t i0 = b * B, i1 = std::min(n, i0 + B);
    std::vector<double> S(&ckpt[b * K * V], &ckpt[b * K * V] + K * V);
    for (int64_t i = i0; i < i1; ++i) {
      step_fwd(K, V, tk, i, S, &Sp_blk[(i - i0) * K * V], &u_blk[(i - i0) * V]);
      std::memcpy(&St_blk[(i - i0) * K * V], S.data(), sizeof(double) * K * V);
    }
    for (int64_t i = i1 - 1; i >= i0; --i) {
      const double* Sp = &Sp_blk[(i - i0) * K * V];
      const double* St = &St_blk[(i - i0) * K * V];
      const double* ut = &u_blk[(i - i0) * V];
      const double* qt = &tk.q[i * K];
      const double* kt = &tk.k[i * K];
      const double* at = &tk.a[i * K];
      const double bt = tk.beta[i];
      const double* dOt = dO + ((t0 + i) * H + h) * V;

      // o_t = scale * S_t^T q_t
      for (int c = 0; c < K; ++c)
        for (int j = 0; j < V; ++j) dS[c * V + j] += P.scale * qt[c] * dOt[j];
      for (int c = 0; c < K; ++c) {
        double acc = 0;
        for (int j = 0; j < V; ++j) acc += St[c * V + j] * dOt[j];
        dqh[i * K + c] = P.scale * acc;
      }
      // S_t = S'_t + beta k u^T
      double db = 0;
      for (int c = 0; c < K; ++c) {
        double acc = 0;
        for (int j = 0; j < V; ++j) acc += dS[c * V + j] * ut[j];
        db += kt[c] * acc;
        dkh[i * K + c] = bt * acc;  // beta * (dS u)
      }
      for (int j = 0; j < V; ++j) {
        double acc = 0;
        for (int c = 0; c < K; ++c) acc += dS[c * V + j] * kt[c];
        du[j] = bt * acc;
      }
      // u_t = v_t - S'^T k_t
      for (int c = 0; c < K; ++c) {
        double acc = 0;
        for (int j = 0; j < V; ++j) acc += Sp[c * V + j] * du[j];
        dkh[i * K + c] -= acc;
      }
      for (int c = 0; c < K; ++c)
        for (int j = 0; j < V; ++j) dSp[c * V + j] = dS[c * V + j] - kt[c] * du[j];
      // S'_t = Diag(exp(g_t)) S_{t-1}
      for (int c = 0; c < K; ++c) {
        double acc = 0;
        for (int j = 0; j < V; ++j) acc += dSp[c * V + j] * Sp[c * V + j];
        dg[i * K + c] = acc;
        for (int j = 0; j < V; ++j) dS[c * V + j] = at[c] * dSp[c * V + j];
      }
      const int64_t t = t0 + i;
      G.dbeta[t * H + h] = db;
      for (int j = 0; j < V; ++j) G.dv[(t * H + h) * V + j] = du[j];
    }
  }

  // dS now holds the gradient w.r.t. the state entering the document
  if (d == 0 && bd.ds_init)
    std::memcpy(bd.ds_init + (int64_t)h * K * V, dS.data(), sizeof(double) * K * V);

  // Chain rule through the L2 norm and the gate transform.
  double dAlog = 0;
  std::vector<double> ddt(K, 0.0);
  for (int64_t i = 0; i < n; ++i) {
    const int64_t t = t0 + i;
    double* dq = G.dq + (t * H + h) * K;
    double* dk = G.dk + (t * H + h) * K;
    if (P.l2norm) {
      double pq = 0, pk = 0;
      for (int c = 0; c < K; ++c) {
        pq += tk.q[i * K + c] * dqh[i * K + c];
        pk += tk.k[i * K + c] * dkh[i * K + c];
      }
      for (int c = 0; c < K; ++c) {
        dq[c] = tk.rq[i] * (dqh[i * K + c] - tk.q[i * K + c] * pq);
        dk[c] = tk.rk[i] * (dkh[i * K + c] - tk.k[i * K + c] * pk);
      }
    } else {
      for (int c = 0; c < K; ++c) {
        dq[c] = dqh[i * K + c];
        dk[c] = dkh[i * K + c];
      }
    }
    double* dgate = G.dgate + (t * H + h) * K;
    if (P.gate_raw) {
      const double* as = in.gate + (t * H + h) * K;
      const double ea = std::exp(in.A_log[h]);
      for (int c = 0; c < K; ++c) {
        const double z = as[c] + in.dt_bias[h * K + c];
        const double dz = dg[i * K + c] * (-ea) * sigmoid(z);
        dgate[c] = dz;
        ddt[c] += dz;
        dAlog += dg[i * K + c] * tk.g[i * K + c];
      }
    } else {
      for (int c = 0; c < K; ++c) dgate[c] = dg[i * K + c];
    }
  }
  if (P.gate_raw) {
    G.dA_log_part[(int64_t)d * H + h] = dAlog;
    for (int c = 0; c < K; ++c) G.ddt_bias_part[((int64_t)d * H + h) * K + c] = ddt[c];
  }
}

int check(const Problem* P, const int64_t* cu) {
  if (!P || !cu) return 1;
  if (P->T < 0 || P->H < 1 || P->N < 0 || P->K < 1 || P->V < 1) return 1;
  if (cu[0] != 0 || cu[P->N] != P->T) return 1;
  for (int d = 0; d < P->N; ++d)
    if (cu[d + 1] < cu[d]) return 1;
  return 0;
}

// Runs fn(d, h) over all (document, head) jobs, longest documents first.
template <class F>
void run_jobs(const Problem& P, const int64_t* cu, int nthreads, F fn) {
  std::vector<std::pair<int64_t, int64_t>> jobs;  // (-len, d*H+h)
  for (int d = 0; d < P.N; ++d)
    for (int h = 0; h < P.H; ++h) jobs.push_back({-(cu[d + 1] - cu[d]), (int64_t)d * P.H + h});
  std::stable_sort(jobs.begin(), jobs.end());
  if (nthreads < 1) nthreads = 1;
  nthreads = (int)std::min<int64_t>(nthreads, std::max<size_t>(jobs.size(), 1));
  std::atomic<size_t> next{0};
  auto worker = [&]() {
    for (;;) {
      size_t j = next.fetch_add(1);
      if (j >= jobs.size()) return;
      int64_t id = jobs[j].second;
      fn((int)(id / P.H), (int)(id % P.H));
    }
  };
  std::vector<std::thread> pool;
  for (int i = 1; i < nthreads; ++i) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

// Forward. o: [T,H,V]. states (nullable): S at the start of every chunk of
// `chunk` tokens, chunks restarting at each document start, ordered by
// document then chunk: [n_chunks, H, K, V] with n_chunks = sum_d ceil(len_d/chunk).
// Returns 0 on success, 1 on invalid arguments.
// s_init, s_final (nullable, [H,K,V]): the state entering document 0 and the
// state leaving the last document.
int kda_oracle_fwd(const Problem* P, const int64_t* cu, const double* q, const double* k,
                   const double* v, const double* beta, const double* gate,
                   const double* A_log, const double* dt_bias, const double* s_init,
                   double* o, double* s_final, double* states, int chunk, int nthreads) {
  if (check(P, cu)) return 1;
  if (P->gate_raw && (!A_log || !dt_bias)) return 1;
  if (states && chunk < 1) return 1;
  Inputs in{cu, q, k, v, beta, gate, A_log, dt_bias};
  std::vector<int64_t> base(P->N + 1, 0);
  for (int d = 0; d < P->N; ++d) {
    int64_t len = cu[d + 1] - cu[d];
    base[d + 1] = base[d] + (states ? (len + chunk - 1) / chunk : 0);
  }
  const Boundary bd{s_init, s_final, nullptr, nullptr};
  if (s_final && P->N == 0) return 1;
  run_jobs(*P, cu, nthreads,
           [&](int d, int h) { fwd_job(*P, in, bd, d, h, o, states, base.data(), chunk); });
  return 0;
}

// Backward of L = sum <o, dO>. dgate receives dg (g form) or da (raw form).
// Raw form also writes dA_log [H] and ddt_bias [H,K], summed over documents
// in document order.
// s_init (nullable): as for the forward; ds_final (nullable): gradient of the
// loss w.r.t. the state leaving the last document; ds_init (nullable) receives
// the gradient w.r.t. s_init.
int kda_oracle_bwd(const Problem* P, const int64_t* cu, const double* q, const double* k,
                   const double* v, const double* beta, const double* gate,
                   const double* A_log, const double* dt_bias, const double* s_init,
                   const double* dO, const double* ds_final, double* dq, double* dk, double* dv,
                   double* dbeta, double* dgate, double* dA_log, double* ddt_bias,
                   double* ds_init, int nthreads) {
  if (check(P, cu)) return 1;
  if (P->gate_raw && (!A_log || !dt_bias || !dA_log || !ddt_bias)) return 1;
  Inputs in{cu, q, k, v, beta, gate, A_log, dt_bias};
  std::vector<double> pA((size_t)P->N * P->H, 0.0), pdt((size_t)P->N * P->H * P->K, 0.0);
  Grads G{dq, dk, dv, dbeta, dgate, pA.data(), pdt.data()};
  const Boundary bd{s_init, nullptr, ds_final, ds_init};
  if (ds_init && P->N == 0) return 1;
  run_jobs(*P, cu, nthreads, [&](int d, int h) { bwd_job(*P, in, bd, dO, G, d, h); });
  if (P->gate_raw) {
    for (int h = 0; h < P->H; ++h) {
      double s = 0;
      for (int d = 0; d < P->N; ++d) s += pA[(size_t)d * P->H + h];
      dA_log[h] = s;
      for (int c = 0; c < P->K; ++c) {
        double t = 0;
        for (int d = 0; d < P->N; ++d) t += pdt[((size_t)d * P->H + h) * P->K + c];
        ddt_bias[h * P->K + c] = t;
      }
    }
  }
  return 0;
}

int kda_oracle_version(void) { return 2; }

}  // extern "C"
