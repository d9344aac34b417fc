// Launch rows of the drop-in optimizers, filled from the parameters in one
// call.  Host code only: it reads tensor metadata (addresses, dtype, layout,
// device) and writes plain integers; it launches nothing and does no
// arithmetic of the method.  The rows are the C ABI's per-tensor structs
// (fo_adamw_tensor, fo_sgdm_tensor in include/foamd.h): pointer and int64
// fields only, so a row of k + 2 fields is k + 2 consecutive int64 words.
#include <torch/extension.h>

#include <cstdint>
#include <vector>

namespace {

// For each parameter i, row i of `dst` becomes (w, fixed[i][0], g,
// fixed[i][1], ..., fixed[i][k-1]) with w the address of the parameter's
// storage and g that of its gradient, `fixed` holding the rest of the row
// (ECC and state addresses, element count).  Returns 0 once every row is
// written, else 1 + the index of the first parameter whose gradient is
// missing, not of dtype `wdt`, not contiguous, on another device or of
// another size; rows from that index on are then not written.  `dst` must
// hold params.size() rows (the caller owns it).
int64_t fill_rows(const std::vector<at::Tensor>& params, const at::Tensor& fixed, int64_t dst,
                  at::ScalarType wdt) {
  TORCH_CHECK(fixed.scalar_type() == at::kLong && fixed.dim() == 2 && fixed.is_contiguous() &&
                  fixed.device().is_cpu(),
              "fixed must be a contiguous int64 CPU matrix");
  TORCH_CHECK(fixed.size(0) == static_cast<int64_t>(params.size()), "one fixed row per parameter");
  TORCH_CHECK(fixed.size(1) >= 2, "a fixed row holds at least the ECC address and the element count");
  TORCH_CHECK(dst != 0, "null destination");
  const int64_t k = fixed.size(1);
  const int64_t* f = fixed.data_ptr<int64_t>();
  int64_t* out = reinterpret_cast<int64_t*>(dst);
  for (size_t i = 0; i < params.size(); ++i) {
    const at::Tensor& p = params[i];
    const at::Tensor& g = p.grad();
    if (!g.defined() || g.scalar_type() != wdt || !g.is_contiguous() || g.device() != p.device() ||
        g.numel() != p.numel())
      return 1 + static_cast<int64_t>(i);
    const int64_t* fi = f + static_cast<int64_t>(i) * k;
    int64_t* r = out + static_cast<int64_t>(i) * (k + 2);
    r[0] = static_cast<int64_t>(reinterpret_cast<intptr_t>(p.data_ptr()));
    r[1] = fi[0];
    r[2] = static_cast<int64_t>(reinterpret_cast<intptr_t>(g.data_ptr()));
    for (int64_t j = 1; j < k; ++j) r[2 + j] = fi[j];
  }
  return 0;
}

}  // namespace

PYBIND11_MODULE(TORCH_EXTENSION_NAME, m) {
  m.doc() = "launch rows of the drop-in optimizers (host code)";
  m.def("fill_rows", &fill_rows, "fill the launch rows of a parameter list (0 = all written)");
}
