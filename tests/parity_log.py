"""Achieved parity errors of the GPU tests, kept per test name so that a drift toward a bar shows.

record(name, err, bar) stores the largest error seen for `name`; the pytest session prints the table at its end
and, when the environment variable SANATAN_PARITY_LOG names a file, writes it there as JSON."""
ERRORS = {}


def record(name, err, bar):
    prev = ERRORS.get(name)
    if prev is None or err > prev["max_err"]:
        ERRORS[name] = {"max_err": float(err), "bar": float(bar), "margin": float(bar / err) if err > 0 else None}
    return err
